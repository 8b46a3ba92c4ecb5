"""Pins of the backward oracle (``oracle.grad``) to what the mathematics fixes.

[D] = "Diagonal Equivalence in State Space Models: Characterization, Retrieval
Rank, and Selective Extensions" (paperpeel.com), Section 2.5 "Parallel scan and
gradients" (the adjoint recurrence) and Appendix C.2 (differentiable carries).

The main pin is independent of the oracle's reverse sweep: central finite
differences of the forward oracle (``ref.scan_seq``) along random directions,
one per input tensor, in fp64.  A dropped term, a wrong sign, a wrong token
index or a transposed operand anywhere in a gradient tensor changes its inner
product with a random direction and fails the comparison.
"""
import math

import numpy as np
import pytest

from m3inputs import make_cotangents, make_small_case
from oracle import grad, ref

_FIELDS = ("x", "B", "C", "dt", "lam", "theta", "B_bias", "C_bias")
_INIT = ("h", "phi", "B_prev", "x_prev")


def _directional(inp, dy, dfin, key, v, sub=None, eps=1e-6):
    """(loss(inp + eps v) - loss(inp - eps v)) / (2 eps) for one tensor."""
    def shifted(s):
        d = dict(inp)
        if sub is None:
            d[key] = np.asarray(inp[key], np.float64) + s * v
        else:
            d[key] = dict(inp[key])
            d[key][sub] = np.asarray(inp[key][sub], np.float64) + s * v
        return d
    return (grad.loss(shifted(eps), dy, dfin) - grad.loss(shifted(-eps), dy, dfin)) / (2.0 * eps)


CASES = [
    # name, kwargs for make_small_case, with final-carry cotangents
    ("static-G=H-R2", dict(batch=2, seqlen=7, nheads=2, headdim=3, dstate=6, rank=2, npairs=2), True),
    ("static-G1-R3-full-turn", dict(batch=1, seqlen=6, nheads=2, ngroups=1, headdim=3, dstate=6, rank=3, npairs=3), True),
    ("heavy-tail", dict(batch=1, seqlen=6, nheads=2, headdim=2, dstate=4, rank=2, npairs=1, rate_dyn=True), True),
    ("siso-no-carry", dict(batch=1, seqlen=5, nheads=1, headdim=3, dstate=4, rank=1, npairs=0, init_full=False,
                           bias=False), False),
    ("one-token", dict(batch=1, seqlen=1, nheads=1, headdim=2, dstate=4, rank=2, npairs=2), True),
]


@pytest.mark.parametrize("name,kw,final", CASES, ids=[c[0] for c in CASES])
def test_gradients_match_finite_differences(name, kw, final):
    """[D] Section 2.5: every gradient (inputs, biases, rate, initial carry)
    equals the directional derivative of the forward recurrence."""
    cfg, inp = make_small_case(70 + len(name), **kw)
    # steps large enough that the decays and turns matter over a few tokens
    inp["dt"] = (np.asarray(inp["dt"], np.float64) * 4.0)
    if inp.get("theta") is not None:
        inp["theta"] = np.asarray(inp["theta"], np.float64) * 8.0
    dy, dfin = make_cotangents(cfg, seed=5, final=final)
    g = grad.scan_bwd(inp, dy, dfin)
    rng = np.random.default_rng(len(name))
    checked = 0
    keys = list(_FIELDS) + (["A_raw"] if inp.get("A_raw") is not None else ["A_log"])
    for key in keys:
        if inp.get(key) is None:
            continue
        v = rng.standard_normal(np.shape(inp[key]))
        fd = _directional(inp, dy, dfin, key, v)
        an = float(np.sum(g[key] * v))
        assert an == pytest.approx(fd, rel=1e-6, abs=1e-7), key
        checked += 1
    if inp.get("init") is not None:
        for sub in _INIT:
            if np.size(inp["init"][sub]) == 0:
                continue
            v = rng.standard_normal(np.shape(inp["init"][sub]))
            fd = _directional(inp, dy, dfin, "init", v, sub=sub)
            an = float(np.sum(g["init"][sub] * v))
            assert an == pytest.approx(fd, rel=1e-6, abs=1e-7), "init." + sub
            checked += 1
    assert checked >= 6


def test_cumulative_sum_adjoint():
    """No decay (A_log = -inf), lambda = 1, dt = 1, no rotation, B = C = e_0:
    y_t is the running sum of x (the forward pin), so d loss / d x_s is the
    reverse running sum of dy over t >= s and d loss / d h0 sums every dy."""
    L, P = 6, 3
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, L, 1, 1, P))
    e0 = np.zeros((1, L, 1, 1, 2))
    e0[..., 0] = 1.0
    inp = {"x": x, "B": e0, "C": e0.copy(), "dt": np.ones((1, L, 1)), "lam": np.ones((1, L, 1)), "theta": None,
           "A_log": np.array([-np.inf]), "B_bias": None, "C_bias": None,
           "init": {"h": np.zeros((1, 1, P, 2)), "phi": np.zeros((1, 1, 0)), "B_prev": np.zeros((1, 1, 1, 2)),
                    "x_prev": np.zeros((1, 1, 1, P))}}
    dy = rng.standard_normal((1, L, 1, 1, P))
    g = grad.scan_bwd(inp, dy)
    want = np.cumsum(dy[0, ::-1, 0, 0], axis=0)[::-1]
    np.testing.assert_allclose(g["x"][0, :, 0, 0], want, rtol=0, atol=1e-14)
    np.testing.assert_allclose(g["init"]["h"][0, 0][:, 0], dy[0, :, 0, 0].sum(axis=0), atol=1e-14)
    np.testing.assert_allclose(g["init"]["h"][0, 0][:, 1], 0.0, atol=0)


def test_rate_gradient_closed_form():
    """P = N = R = 1, one token, no carry but h0: y = exp(-dt a) h0 C, so
    d y / d A_log = -dt a y (a = exp(A_log)) and d y / d dt = -a y + lam C x."""
    a_log, dt, lam, h0, xv, cv = 0.3, 0.7, 0.4, 1.3, -0.8, 1.1
    inp = {"x": np.full((1, 1, 1, 1, 1), xv), "B": np.ones((1, 1, 1, 1, 1)), "C": np.full((1, 1, 1, 1, 1), cv),
           "dt": np.full((1, 1, 1), dt), "lam": np.full((1, 1, 1), lam), "theta": None,
           "A_log": np.array([a_log]), "B_bias": None, "C_bias": None,
           "init": {"h": np.full((1, 1, 1, 1), h0), "phi": np.zeros((1, 1, 0)), "B_prev": np.zeros((1, 1, 1, 1)),
                    "x_prev": np.zeros((1, 1, 1, 1))}}
    a = math.exp(a_log)
    decayed = math.exp(-dt * a) * h0 * cv
    g = grad.scan_bwd(inp, np.ones((1, 1, 1, 1, 1)))
    assert g["A_log"][0] == pytest.approx(-dt * a * decayed, rel=1e-13)
    assert g["dt"][0, 0, 0] == pytest.approx(-a * decayed + lam * cv * xv, rel=1e-13)
    assert g["lam"][0, 0, 0] == pytest.approx(dt * cv * xv, rel=1e-13)


def test_heavy_tail_rate_grad():
    """The rate law's derivative: -1 above zero, -1/(1-u)^2 below, 0 in the clamp."""
    u = np.array([2.0, 0.0, -1.0, -3.0, -2e4])
    np.testing.assert_allclose(grad.heavy_tail_rate_grad(u), [-1.0, -1.0, -0.25, -1.0 / 16.0, 0.0], rtol=1e-15)
    h = 1e-7
    for v in (0.7, -0.4, -5.0):
        fd = (ref.heavy_tail_rate(v + h) - ref.heavy_tail_rate(v - h)) / (2 * h)
        assert grad.heavy_tail_rate_grad(v) == pytest.approx(float(fd), rel=1e-7)


def test_angle_invariance_single_token():
    """[M3] "Computing the rotation as a data-dependent RoPE": B and C turn by the same
    angle, so with one token and no carry every C . B product is unchanged by it and
    the angle gradients are zero (here to fp64 rounding), while the B, C gradients are not."""
    cfg, inp = make_small_case(8, batch=1, seqlen=1, nheads=2, headdim=3, dstate=8, rank=2, npairs=4,
                               init_full=False)
    dy, _ = make_cotangents(cfg, seed=2, final=False)
    g = grad.scan_bwd(inp, dy)
    scale = float(np.abs(g["B"]).max())
    assert scale > 1e-3
    assert float(np.abs(g["theta"]).max()) <= 1e-13 * scale
    assert float(np.abs(g["init"]["phi"]).max()) <= 1e-13 * scale
