"""Pins of the per-coordinate scan oracle (``oracle.pcs``), each against
something other than the oracle's own recurrence: the scalar-decay oracle of the
Mamba-3 scan, numpy's running sum, a closed-form geometric series, brute force
over token pairs, and invariances.  A planted slip in the recurrence is caught."""
import numpy as np

from m3inputs.pcs import make_pcs_inputs
from oracle import pcs, ref


def _small(seed, **kw):
    args = dict(batch=2, channels=6, seqlen=13, dstate=5, ngroups=2, io="f32", seed=seed, init=True)
    args.update(kw)
    return make_pcs_inputs(**args)


def test_sequential_equals_quadratic_and_associative():
    """The recurrence, the sum over token pairs with one decay mask per
    coordinate, and the prefix of the associative combine agree (brute force)."""
    for seed, kw in ((1, {}), (2, dict(ngroups=1, dstate=1)), (3, dict(channels=4, ngroups=4, seqlen=1)),
                     (4, dict(init=False, seqlen=20))):
        d = _small(seed, **kw)
        y, h = pcs.scan_seq(d, d["h0"])
        yq = pcs.scan_quadratic(d, d["h0"])
        ya, ha = pcs.scan_assoc(d, d["h0"])
        assert np.allclose(y, yq, rtol=1e-12, atol=1e-12)
        assert np.allclose(y, ya, rtol=1e-12, atol=1e-12) and np.allclose(h, ha, rtol=1e-12, atol=1e-12)


def test_equal_decay_rows_reduce_to_the_scalar_decay_scan():
    """With every coordinate of a channel decaying at one rate, each channel is a
    one-channel head of the scalar-decay scan with the rectangle write (rank 1, no
    rotation, lambda = 1: gamma = dt, no lagged term), computed by the Mamba-3
    oracle ``ref.scan_seq``."""
    d = _small(5, channels=4, ngroups=2, dstate=6)
    row = np.log(np.random.default_rng(0).uniform(1, 16, size=4)).astype(np.float32)
    d["A_log"] = np.repeat(row[:, None], 6, axis=1)
    y, h = pcs.scan_seq(d, d["h0"])
    b, L, D = d["x"].shape
    inp = {"x": d["x"][:, :, :, None, None], "B": d["B"][:, :, :, None, :], "C": d["C"][:, :, :, None, :],
           "dt": d["dt"], "lam": np.ones_like(d["dt"]), "theta": None, "A_log": row, "B_bias": None,
           "C_bias": None, "init": {"h": d["h0"][:, :, None, :], "phi": np.zeros((b, D, 0)),
                                    "B_prev": np.zeros((b, D, 1, 6)), "x_prev": np.zeros((b, D, 1, 1))}}
    yr, fr = ref.scan_seq(inp)
    assert np.allclose(y, yr[:, :, :, 0, 0], rtol=1e-12, atol=1e-12)
    assert np.allclose(h, fr["h"][:, :, 0, :], rtol=1e-12, atol=1e-12)


def test_no_decay_gives_the_running_sum():
    """a = 0 (alpha = 1), dt = 1, B = C = e_0: y is numpy's running sum of x."""
    d = _small(6, ngroups=1, init=False)
    d["A_log"][:] = -np.inf
    d["dt"][:] = 1.0
    d["B"][:] = 0.0
    d["C"][:] = 0.0
    d["B"][..., 0] = 1.0
    d["C"][..., 0] = 1.0
    y, _ = pcs.scan_seq(d)
    assert np.allclose(y, np.cumsum(d["x"].astype(np.float64), axis=1), rtol=1e-12, atol=1e-12)


def test_impulse_gives_the_geometric_series():
    """One coordinate, constant step s and rate a, B = C = 1, x an impulse at
    t = 0: y_t = s exp(s a t) (the write has gain s, each step decays by exp(s a))."""
    L, s, a = 40, 0.3, -1.7
    d = _small(7, batch=1, channels=1, ngroups=1, dstate=1, seqlen=L, init=False)
    d["A_log"][:] = np.log(-a)
    d["dt"][:] = s
    d["B"][:] = 1.0
    d["C"][:] = 1.0
    d["x"][:] = 0.0
    d["x"][0, 0, 0] = 1.0
    y, h = pcs.scan_seq(d)
    t = np.arange(L)
    want = np.float32(s) * np.exp(np.float64(np.float32(s)) * (-np.exp(np.float64(np.float32(np.log(-a))))) * t)
    assert np.allclose(y[0, :, 0], want, rtol=1e-12, atol=1e-15)
    assert np.isclose(h[0, 0, 0], want[-1], rtol=1e-12)


def test_planted_slip_is_caught():
    """A plausible mistake -- the decay applied after the write instead of before it
    -- fails the geometric-series pin."""
    L, s, a = 10, 0.3, -1.7
    d = _small(8, batch=1, channels=1, ngroups=1, dstate=1, seqlen=L, init=False)
    d["A_log"][:] = np.log(-a)
    d["dt"][:] = s
    d["B"][:] = 1.0
    d["C"][:] = 1.0
    d["x"][:] = 0.0
    d["x"][0, 0, 0] = 1.0
    h, wrong = 0.0, []
    for t in range(L):                      # slip: h = alpha (h + dt B x)
        al = np.exp(np.float64(d["dt"][0, t, 0]) * -np.exp(np.float64(d["A_log"][0, 0])))
        h = al * (h + np.float64(d["dt"][0, t, 0]) * d["x"][0, t, 0])
        wrong.append(h)
    y, _ = pcs.scan_seq(d)
    assert not np.allclose(np.array(wrong), y[0, :, 0], rtol=1e-6)


def test_coordinate_permutation_superposition_and_continuation():
    """Coordinates are independent (permuting n in A, B, C together leaves y
    unchanged); y is linear in (h0, x); a split sequence with the state carried
    equals the whole."""
    d = _small(9, seqlen=17)
    y, h = pcs.scan_seq(d, d["h0"])
    perm = np.random.default_rng(1).permutation(d["A_log"].shape[1])
    dp = dict(d, A_log=d["A_log"][:, perm], B=d["B"][..., perm], C=d["C"][..., perm])
    yp, hp = pcs.scan_seq(dp, d["h0"][..., perm])
    assert np.allclose(y, yp, rtol=1e-12, atol=1e-12) and np.allclose(h[..., perm], hp, rtol=1e-12, atol=1e-12)
    y0, _ = pcs.scan_seq(d, None)
    yh, _ = pcs.scan_seq(dict(d, x=np.zeros_like(d["x"])), d["h0"])
    assert np.allclose(y, y0 + yh, rtol=1e-12, atol=1e-12)
    cut = 7
    sl = lambda a, i, j: a[:, i:j]  # noqa: E731
    d1 = dict(d, x=sl(d["x"], 0, cut), dt=sl(d["dt"], 0, cut), B=sl(d["B"], 0, cut), C=sl(d["C"], 0, cut))
    d2 = dict(d, x=sl(d["x"], cut, None), dt=sl(d["dt"], cut, None), B=sl(d["B"], cut, None), C=sl(d["C"], cut, None))
    y1, h1 = pcs.scan_seq(d1, d["h0"])
    y2, h2 = pcs.scan_seq(d2, h1)
    assert np.allclose(np.concatenate([y1, y2], axis=1), y, rtol=1e-12, atol=1e-12)
    assert np.allclose(h2, h, rtol=1e-12, atol=1e-12)


def test_c_oracle_equals_numpy():
    """The C recurrence (used at full size) equals the numpy one to rounding, on
    all channels and on a channel range."""
    from oracle import pcs_cpu
    d = _small(10, channels=8, ngroups=4, seqlen=30)
    y, h = pcs.scan_seq(d, d["h0"])
    yc, hc = pcs_cpu.scan(d, d["h0"])
    assert np.allclose(yc, y, rtol=1e-12, atol=1e-12) and np.allclose(hc, h, rtol=1e-12, atol=1e-12)
    yr, hr = pcs_cpu.scan(d, d["h0"], 3, 7)
    assert np.allclose(yr, y[:, :, 3:7], rtol=1e-12, atol=1e-12) and np.allclose(hr, h[:, 3:7], rtol=1e-12, atol=1e-12)
    y0, _ = pcs_cpu.scan(d, None)
    yn, _ = pcs.scan_seq(d, None)
    assert np.allclose(y0, yn, rtol=1e-12, atol=1e-12)
