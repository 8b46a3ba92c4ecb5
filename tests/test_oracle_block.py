"""Pins of the layer-step oracle (``oracle.block``) to closed forms, identities
and the scan oracle.

[M3] = "Mamba-3: Improved Sequence Modeling using State Space Principles"
(intuitivepapers.ai): the decode listing of "Computing the rotation as a
data-dependent RoPE", "MIMO: a rank-4 state update", "The Mamba-3 block, layer
by layer".
"""
import json
import math
import os

import numpy as np
import pytest

from m3inputs import config_by_name, make_block_inputs
from oracle import block, ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def _case(seed=5, R=2, npairs=2, L=11, G=1, N=8, P=4, H=2, b=2):
    cfg = config_by_name("tiny_siso_f32").with_(batch=b, seqlen=L, nheads=H, ngroups=G, headdim=P, dstate=N,
                                                rank=R, npairs=npairs)
    return cfg, make_block_inputs(cfg, seed=seed)


# --------------------------------------------------------------------------
# activations and the norm
# --------------------------------------------------------------------------
def test_activations_closed_forms():
    """[M3] decode listing and the remarks after it: softplus on the step,
    sigmoid on lambda, silu on the gate, pi tanh on the angle."""
    assert block.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    assert block.softplus(40.0) == pytest.approx(40.0, rel=1e-15)
    assert block.softplus(-40.0) == pytest.approx(math.exp(-40.0), rel=1e-12)
    v = np.linspace(-20.0, 20.0, 401)
    assert np.allclose(block.softplus(v) - block.softplus(-v), v, rtol=0, atol=1e-12)      # log(e^v) = v
    assert np.allclose(np.exp(block.softplus(v)), 1.0 + np.exp(v), rtol=1e-12)
    assert block.sigmoid(0.0) == 0.5
    assert np.allclose(block.sigmoid(v) + block.sigmoid(-v), 1.0, atol=1e-15)
    assert np.allclose(block.sigmoid(v), 1.0 / (1.0 + np.exp(-v)), rtol=1e-13)
    assert block.silu(0.0) == 0.0
    assert np.allclose(block.silu(v) - block.silu(-v), v, atol=1e-12)                      # v (s(v) + s(-v)) = v
    assert block.angle_rate(0.0) == 0.0
    assert block.angle_rate(50.0) == pytest.approx(math.pi, rel=1e-15)
    assert np.allclose(block.angle_rate(-v), -block.angle_rate(v))
    assert np.all(np.abs(block.angle_rate(v)) <= math.pi)


def test_rms_norm():
    """[M3] "The Mamba-3 block": BCNorm gives unit root-mean-square entries."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal((5, 128)) * 7.0
    out = block.rms_norm(v, eps=0.0)
    assert np.allclose(np.sqrt(np.mean(out * out, axis=-1)), 1.0, atol=1e-14)
    assert np.allclose(block.rms_norm(3.5 * v, eps=0.0), out, atol=1e-14)                  # scale invariant
    assert np.allclose(block.rms_norm(-v, eps=0.0), -out, atol=1e-14)
    g = rng.standard_normal(128)
    assert np.allclose(block.rms_norm(v, g, eps=0.0), out * g, atol=1e-14)
    assert np.all(block.rms_norm(np.zeros((2, 8))) == 0.0)                                # eps keeps 0 at 0


# --------------------------------------------------------------------------
# the layer against the page's worked example and the scan oracle
# --------------------------------------------------------------------------
def _scalar_block(xs, lams, dts, us, z):
    """P = N = R = H = 1, one group; raw inputs whose activations are the
    given values (inverses written from the closed forms)."""
    L = len(xs)
    one = lambda v: np.asarray(v, np.float64).reshape(1, L, 1)  # noqa: E731
    params = {"dt_bias": np.zeros(1), "B_gain": None, "C_gain": None, "lift": np.ones((1, 1, 1)),
              "comb": np.ones((1, 1, 1)), "D": None, "B_bias": None, "C_bias": None}
    return {"z": np.full((1, L, 1, 1), z), "x": np.asarray(xs, np.float64).reshape(1, L, 1, 1),
            "B_raw": np.ones((1, L, 1, 1, 1)), "C_raw": np.ones((1, L, 1, 1, 1)),
            "dt_raw": one(np.log(np.expm1(dts))), "A_raw": one(us),
            "lam_raw": one(np.log(np.asarray(lams) / (1.0 - np.asarray(lams)))), "th_raw": None,
            "params": params, "init": None}


def test_worked_example_through_the_layer():
    """[M3] "How the exponential-trapezoidal update works": dt = 0.5, A = -1
    (rate input 0), lambda = 0.7, x = (1, 0, 0) gives 0.35, 0.303, 0.184 for
    the readout; B = C = 1 after the norm (up to its eps), gate 1."""
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    zstar = 1.0                                   # silu(z*) = 1: z* / (1 + exp(-z*)) = 1
    for _ in range(60):
        zstar = 1.0 + math.exp(-zstar)
    out, _ = block.block_forward(_scalar_block([1.0, 0.0, 0.0], [0.7] * 3, [0.5] * 3, [0.0] * 3, zstar))
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    np.testing.assert_allclose(out.reshape(-1), g["mamba3_states"], atol=tol)
    e = math.exp(-0.5)
    np.testing.assert_allclose(out.reshape(-1), [0.35, 0.5 * e, 0.5 * e * e], rtol=1e-5)


@pytest.mark.parametrize("seed,R,npairs", [(11, 1, 0), (12, 2, 2), (13, 4, 3)])
def test_layer_is_scan_of_activated_inputs(seed, R, npairs):
    """The layer equals the scan oracle run on inputs built from the closed-form
    inverses of the activations (softplus^-1, logit, atanh), with unit-RMS raw B
    and C (so the norm only divides by sqrt(1 + eps)), one-hot readout weights
    and no skip, gated by silu(z) computed here."""
    cfg, d = _case(seed, R=R, npairs=npairs)
    rng = np.random.default_rng(seed)
    b, L, H, P = d["x"].shape
    G, N = d["B_raw"].shape[2], d["B_raw"].shape[4]
    Bn = rng.standard_normal((b, L, G, R, N))
    Bn /= np.sqrt(np.mean(Bn * Bn, axis=-1, keepdims=True))
    Cn = rng.standard_normal((b, L, G, R, N))
    Cn /= np.sqrt(np.mean(Cn * Cn, axis=-1, keepdims=True))
    dt = rng.uniform(0.05, 0.8, size=(b, L, H))
    lam = rng.uniform(0.05, 0.95, size=(b, L, H))
    th = rng.uniform(-2.5, 2.5, size=(b, L, H, npairs))
    r_sel = R - 1
    comb = np.zeros((H, R, P))
    comb[:, r_sel, :] = 1.0
    d.update(B_raw=Bn, C_raw=Cn, dt_raw=np.log(np.expm1(dt)) - d["params"]["dt_bias"][None, None, :],
             lam_raw=np.log(lam / (1.0 - lam)), th_raw=np.arctanh(th / math.pi) if npairs else None)
    d["params"] = dict(d["params"], B_gain=None, C_gain=None, comb=comb, D=None)
    out, fin = block.block_forward(d)
    shrink = 1.0 / math.sqrt(1.0 + block.RMS_EPS)          # unit-RMS rows through the norm's eps
    scan_in = {"x": np.asarray(d["x"], np.float64)[:, :, :, None, :] * np.asarray(d["params"]["lift"])[None, None],
               "B": Bn * shrink, "C": Cn * shrink, "dt": dt, "lam": lam, "theta": th if npairs else None, "A_log": None,
               "A_raw": d["A_raw"], "B_bias": d["params"]["B_bias"], "C_bias": d["params"]["C_bias"],
               "init": d["init"]}
    y, f2 = ref.scan_seq(scan_in)
    z = np.asarray(d["z"], np.float64)
    gate = z / (1.0 + np.exp(-z))
    assert _rel(out, y[:, :, :, r_sel, :] * gate) < 1e-12
    assert _rel(fin["h"], f2["h"]) < 1e-12


def test_linear_in_the_lift():
    """Without the skip, the output is linear in the x lift (the scan is linear
    in x for fixed B, C and decays)."""
    _, d = _case(21, R=2)
    d["params"] = dict(d["params"], D=None)
    d["init"] = None
    o1, _ = block.block_forward(d)
    d2 = dict(d, params=dict(d["params"], lift=2.5 * np.asarray(d["params"]["lift"], np.float64)))
    o2, _ = block.block_forward(d2)
    assert _rel(o2, 2.5 * o1) < 1e-12


def test_skip_and_gate_closed_form():
    """[M3] decode listing: y = h C + D x, output y silu(z).  With C = 0 (raw C
    and its bias zero) every readout vanishes and the output is D x silu(z),
    with the un-lifted x (the lift is 2 here)."""
    _, d = _case(31, R=2)
    d["C_raw"] = np.zeros_like(d["C_raw"])
    d["params"] = dict(d["params"], C_bias=None, lift=2.0 * np.ones_like(d["params"]["lift"]))
    out, _ = block.block_forward(d)
    z = np.asarray(d["z"], np.float64)
    want = np.asarray(d["params"]["D"], np.float64)[None, None, :, None] * d["x"] * z / (1.0 + np.exp(-z))
    assert _rel(out, want) < 1e-14


def test_bias_after_the_norm():
    """[M3] "The Mamba-3 block": the bias is added after the norm, so scaling the
    raw B and C leaves the layer unchanged while scaling the bias does not."""
    _, d = _case(41, R=2, npairs=2)
    o1, _ = block.block_forward(d)
    o2, _ = block.block_forward(dict(d, B_raw=7.0 * d["B_raw"], C_raw=0.2 * d["C_raw"]))
    assert _rel(o2, o1) < 1e-6                      # the norm's eps only
    o3, _ = block.block_forward(dict(d, params=dict(d["params"], B_bias=2.0 * d["params"]["B_bias"])))
    assert _rel(o3, o1) > 1e-2


def test_decode_steps_equal_layer():
    """[M3] decode listing: token-by-token layer steps (carry: state, phase,
    previous biased and turned B, previous lifted x) equal the whole-sequence
    layer."""
    _, d = _case(51, R=2, npairs=2, L=9)
    out, fin = block.block_forward(d)
    carry = {k: np.asarray(v, np.float64) for k, v in d["init"].items()}
    outs = []
    for t in range(9):
        tok = {k: d[k][:, t] for k in ("z", "x", "B_raw", "C_raw", "dt_raw", "A_raw", "lam_raw")}
        tok["th_raw"] = d["th_raw"][:, t]
        o, carry = block.block_decode_step(carry, tok, d["params"])
        outs.append(o)
    assert _rel(np.stack(outs, axis=1), out) < 1e-12
    assert _rel(carry["h"], fin["h"]) < 1e-12
    assert _rel(carry["x_prev"], fin["x_prev"]) < 1e-12


def test_planted_skip_on_lifted_x_is_caught(monkeypatch):
    """A slip that adds D times the lifted x (rank 0 copy) fails the closed form."""
    _, d = _case(31, R=2)
    d["C_raw"] = np.zeros_like(d["C_raw"])
    d["params"] = dict(d["params"], C_bias=None, lift=2.0 * np.ones_like(d["params"]["lift"]))
    good, _ = block.block_forward(d)
    orig = block.epilogue

    def bad(blk, y):
        b2 = dict(blk, x=2.0 * np.asarray(blk["x"]))
        return orig(b2, y)
    monkeypatch.setattr(block, "epilogue", bad)
    wrong, _ = block.block_forward(d)
    assert _rel(wrong, good) > 0.5
