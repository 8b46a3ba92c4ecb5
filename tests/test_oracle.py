"""Pins of the CPU oracle to what the pages and the mathematics fix.

Each test names the passage it follows.  [M3] = "Mamba-3: Improved Sequence
Modeling using State Space Principles" (intuitivepapers.ai); [D] = "Diagonal
Equivalence in State Space Models: Characterization, Retrieval Rank, and
Selective Extensions" (paperpeel.com).
"""
import json
import math
import os

import numpy as np
import pytest

from m3inputs import make_small_case
from oracle import model, ref, ref_cpu

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def _case_scalar(dts, lams, xs, A_log=0.0):
    """P = N = R = 1, B = C = 1, no rotation (the worked example's setting)."""
    L = len(xs)
    return {
        "x": np.array(xs, np.float32).reshape(1, L, 1, 1, 1),
        "B": np.ones((1, L, 1, 1, 1), np.float32),
        "C": np.ones((1, L, 1, 1, 1), np.float32),
        "dt": np.array(dts, np.float32).reshape(1, L, 1),
        "lam": np.array(lams, np.float32).reshape(1, L, 1),
        "theta": None, "A_log": np.array([A_log], np.float32),
        "B_bias": None, "C_bias": None, "init": None,
    }


ALL_FORMS = {
    "seq": ref.scan_seq,
    "quadratic": ref.scan_quadratic,
    "chunked2": lambda d: ref.scan_chunked(d, 2),
    "unrotated": ref.scan_seq_unrotated,
    "c": lambda d: ref_cpu.scan(d),
}


# --------------------------------------------------------------------------
# pin 1: the worked example
# --------------------------------------------------------------------------
@pytest.mark.parametrize("form", sorted(ALL_FORMS))
def test_worked_example(form):
    """[M3] "How the exponential-trapezoidal update works", worked step:
    dt = 0.5, A = -1, lam = 0.7, x = (1, 0, 0), B = 1 -> 0.35, 0.303, 0.184;
    Mamba-2 (lam = 1) -> 0.500, 0.303, 0.184; a second token with lam = 0.2
    leaves 0.455 -- which fixes that the lagged term is weighted by the
    *later* token's lam and dt."""
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    s = g["setup"]
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    f = ALL_FORMS[form]
    y, _ = f(_case_scalar([s["dt"]] * 3, [s["lam"]] * 3, s["x"], s["A_log"]))
    np.testing.assert_allclose(y.reshape(-1), g["mamba3_states"], atol=tol)
    y2, _ = f(_case_scalar([s["dt"]] * 3, [1.0] * 3, s["x"], s["A_log"]))
    np.testing.assert_allclose(y2.reshape(-1), g["mamba2_states"], atol=tol)
    y3, _ = f(_case_scalar([s["dt"]] * 3, [s["lam"], 0.2, s["lam"]], s["x"], s["A_log"]))
    assert abs(y3.reshape(-1)[1] - g["second_token_lam_0p2"]["state_after_second"]) <= tol
    # the exact values behind the printed ones
    e = math.exp(-0.5)
    np.testing.assert_allclose(y.reshape(-1), [0.35, 0.5 * e, 0.5 * e * e], rtol=1e-6)
    assert abs(y3.reshape(-1)[1] - 0.75 * e) < 1e-6


def test_worked_example_coefficients():
    """The page's alpha = 0.607, gamma = 0.35, beta = 0.091 for the same step,
    recovered from the decode step by feeding unit impulses."""
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    carry = {"h": np.ones((1, 1, 1, 1)), "phi": np.zeros((1, 1, 0)),
             "B_prev": np.zeros((1, 1, 1, 1)), "x_prev": np.zeros((1, 1, 1, 1))}
    one = np.ones((1, 1, 1, 1))
    args = dict(B=one, C=one, dt=np.full((1, 1), 0.5), lam=np.full((1, 1), 0.7),
                theta=None, A_log=np.zeros(1))
    ya, _ = ref.decode_step(carry, x=np.zeros((1, 1, 1, 1)), **args)            # alpha * 1
    c0 = dict(carry, h=np.zeros((1, 1, 1, 1)))
    yg, _ = ref.decode_step(c0, x=one, **args)                                  # gamma * 1
    c1 = dict(c0, B_prev=one, x_prev=one)
    yb, _ = ref.decode_step(c1, x=np.zeros((1, 1, 1, 1)), **args)               # beta * 1
    assert abs(ya.item() - g["alpha"]) < 5e-4
    assert abs(yg.item() - g["gamma"]) < 5e-4
    assert abs(yb.item() - g["beta"]) < 5e-4


# --------------------------------------------------------------------------
# pin 2: brute-force quadratic = sequential = chunked (every chunk size)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed,R,npairs,N,G,L", [
    (1, 1, 0, 4, 2, 9), (2, 2, 1, 4, 1, 13), (3, 3, 2, 4, 2, 11),
    (4, 4, 3, 6, 1, 12), (5, 2, 2, 5, 2, 10),
])
def test_quadratic_sequential_chunked(seed, R, npairs, N, G, L):
    """[M3] "The trapezoid term as a two-tap filter" (mask = decay mask x
    bidiagonal band), "MIMO" (R^2 cross terms), [D] 2.4 (chunk-local
    cumulative log-decays, carried boundary state), with nonzero carries and
    chunk sizes that do and do not divide L."""
    _, d = make_small_case(seed, batch=2, seqlen=L, nheads=2, ngroups=G, headdim=3,
                           dstate=N, rank=R, npairs=npairs, init_full=True, dt_scale=3.0)
    y0, f0 = ref.scan_seq(d)
    yq, fq = ref.scan_quadratic(d)
    assert _rel(yq, y0) < 1e-12
    for k in ("h", "B_prev", "x_prev"):
        assert _rel(fq[k], f0[k]) < 1e-12
    for q in range(1, L + 1):
        yc, fc = ref.scan_chunked(d, q)
        assert _rel(yc, y0) < 1e-12, q
        assert _rel(fc["h"], f0["h"]) < 1e-12, q
        assert _rel(fc["B_prev"], f0["B_prev"]) < 1e-12
    assert np.allclose(np.cos(fq["phi"]), np.cos(f0["phi"]), atol=1e-12)


# --------------------------------------------------------------------------
# pin 3: reduction to Mamba-2 scalar SSD
# --------------------------------------------------------------------------
def test_mamba2_reduction():
    """[M3] "How Mamba gets its recurrence ..." and "How the exponential-
    trapezoidal update works": with lam = 1 the middle term vanishes and the
    update is Mamba-2's h_t = exp(dt_t A) h_{t-1} + dt_t x_t B_t, y_t = h_t C_t;
    the SSD mask is prod(alpha) * dt_s ("The trapezoid term as a two-tap
    filter").  R = 1, no rotation."""
    cfg, d = make_small_case(11, batch=1, seqlen=17, nheads=3, ngroups=1, headdim=4,
                             dstate=5, rank=1, npairs=0, bias=False, lam_one=True,
                             init_full=False, dt_scale=2.0)
    y, _ = ref.scan_seq(d)
    x = d["x"][0, :, :, 0, :].astype(np.float64)        # [L,H,P]
    Bm = d["B"][0, :, 0, 0, :].astype(np.float64)       # [L,N]
    Cm = d["C"][0, :, 0, 0, :].astype(np.float64)
    for h in range(3):
        A = -math.exp(float(d["A_log"][h]))
        dt = d["dt"][0, :, h].astype(np.float64)
        # (a) the three-line recurrence
        hs, ys = np.zeros((4, 5)), []
        for t in range(17):
            hs = math.exp(dt[t] * A) * hs + dt[t] * np.outer(x[t, h], Bm[t])
            ys.append(hs @ Cm[t])
        assert _rel(y[0, :, h, 0, :], np.array(ys)) < 1e-12
        # (b) the scalar SSD masked form with segment sums
        cs = np.concatenate([[0.0], np.cumsum(dt * A)])
        Lm = np.array([[math.exp(cs[t + 1] - cs[s + 1]) * dt[s] if s <= t else 0.0
                        for s in range(17)] for t in range(17)])
        ssd = (Lm * (Cm @ Bm.T)) @ x[:, h]
        assert _rel(y[0, :, h, 0, :], ssd) < 1e-12


# --------------------------------------------------------------------------
# pin 4: alpha = 1, theta = 0 cumulative-sum invariant
# --------------------------------------------------------------------------
@pytest.mark.parametrize("form", sorted(ALL_FORMS))
def test_cumsum_invariant(form):
    """No decay (A_log = -inf gives alpha = 1), lam = 1, dt = 1, no rotation:
    y_t = sum_{s<=t} (C_t . B_s) x_s; with B = C = e_0 for every rank, every
    readout is the running sum of x over time and ranks (numpy.cumsum)."""
    L, R, P, N = 12, 3, 5, 4
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, L, 1, R, P)).astype(np.float32)
    e0 = np.zeros((1, L, 1, R, N), np.float32)
    e0[..., 0] = 1.0
    d = {"x": x, "B": e0, "C": e0.copy(), "dt": np.ones((1, L, 1), np.float32),
         "lam": np.ones((1, L, 1), np.float32), "theta": None,
         "A_log": np.array([-np.inf], np.float32), "B_bias": None, "C_bias": None, "init": None}
    y, _ = ALL_FORMS[form](d)
    want = np.cumsum(x.astype(np.float64).sum(axis=3), axis=1)   # [1,L,1,P]
    for r in range(R):
        assert _rel(y[:, :, :, r, :], want) < 1e-12
    # and with general B, C: the plain causal sum of (C_t . B_s) x_s
    B = rng.standard_normal((1, L, 1, R, N)).astype(np.float32)
    C = rng.standard_normal((1, L, 1, R, N)).astype(np.float32)
    d.update(B=B, C=C)
    y, _ = ALL_FORMS[form](d)
    for t in range(L):
        for r in range(R):
            acc = sum(float(C[0, t, 0, r].astype(np.float64) @ B[0, s, 0, q].astype(np.float64))
                          * x[0, s, 0, q].astype(np.float64)
                      for s in range(t + 1) for q in range(R))
            assert np.allclose(y[0, t, 0, r], acc, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# pin 5: rotated-B/C form = rotating-state form
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [21, 22, 23])
def test_rotated_equals_unrotated(seed):
    """[M3] "Computing the rotation as a data-dependent RoPE": turning B and C
    by the running rotation (the lagged term keeping the previous token's
    rotation) gives the same outputs as turning the state every step."""
    _, d = make_small_case(seed, batch=1, seqlen=14, nheads=2, ngroups=1, headdim=3,
                           dstate=8, rank=2, npairs=4, init_full=True)
    d["theta"] = (d["theta"] * 300.0).astype(np.float32)   # large turns per step
    y0, f0 = ref.scan_seq(d)
    y1, f1 = ref.scan_seq_unrotated(d)
    assert _rel(y1, y0) < 1e-12
    assert _rel(f1["h"], f0["h"]) < 1e-12
    assert _rel(f1["B_prev"], f0["B_prev"]) < 1e-12


# --------------------------------------------------------------------------
# pin 6: dt = 1, constant theta is ordinary RoPE
# --------------------------------------------------------------------------
def test_rope_reduction():
    """[M3] "Computing the rotation as a data-dependent RoPE": with dt = 1 and a
    constant theta the read-write weight is C_t^T Rot((s - t) theta) B_s per
    pair, a function of t - s only -- ordinary rotary embedding.  Checked with
    complex arithmetic: pair i as the complex number v_2i + i v_2i+1, rotated
    by multiplying with exp(i * angle)."""
    L, N, npairs = 10, 6, 2
    rng = np.random.default_rng(3)
    freqs = np.array([0.7, 0.11])
    B = rng.standard_normal((1, L, 1, 1, N)).astype(np.float32)
    C = rng.standard_normal((1, L, 1, 1, N)).astype(np.float32)
    x = rng.standard_normal((1, L, 1, 1, 1)).astype(np.float32)
    d = {"x": x, "B": B, "C": C, "dt": np.ones((1, L, 1), np.float32),
         "lam": np.ones((1, L, 1), np.float32),
         "theta": np.broadcast_to(freqs.astype(np.float32), (1, L, 1, npairs)).copy(),
         "A_log": np.array([-np.inf], np.float32), "B_bias": None, "C_bias": None, "init": None}
    y, _ = ref.scan_seq(d)
    th = d["theta"][0, 0, 0].astype(np.float64)
    Bz = B[0, :, 0, 0].astype(np.float64)
    Cz = C[0, :, 0, 0].astype(np.float64)
    bz = Bz[:, 0:4:2] + 1j * Bz[:, 1:4:2]
    cz = Cz[:, 0:4:2] + 1j * Cz[:, 1:4:2]
    for t in range(L):
        acc = 0.0
        for s in range(t + 1):
            w = np.sum((np.conj(cz[t]) * bz[s] * np.exp(1j * (s - t) * th)).real)
            w += Cz[t, 4:] @ Bz[s, 4:]
            acc += w * float(x[0, s, 0, 0, 0])
        assert abs(y[0, t, 0, 0, 0] - acc) < 1e-12 * max(1.0, abs(acc))
    # shift invariance: the weight of a (t, s) pair depends on t - s only
    e = np.zeros((1, L, 1, 1, 1), np.float32)
    e[0, 0] = 1.0
    Bc = np.broadcast_to(B[:, :1], B.shape).copy()
    Cc = np.broadcast_to(C[:, :1], C.shape).copy()
    d1 = dict(d, x=e, B=Bc, C=Cc)
    y1, _ = ref.scan_seq(d1)
    e2 = np.zeros_like(e)
    e2[0, 3] = 1.0
    y2, _ = ref.scan_seq(dict(d1, x=e2))
    np.testing.assert_allclose(y2[0, 3:, 0, 0, 0], y1[0, :L - 3, 0, 0, 0], rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# pin 7: parity and mod-5 counting with a rotating state
# --------------------------------------------------------------------------
def _counter(bits, angle):
    L = len(bits)
    x = np.zeros((1, L, 1, 1, 1), np.float32)
    x[0, 0] = 1.0
    e0 = np.zeros((1, L, 1, 1, 2), np.float32)
    e0[..., 0] = 1.0
    th = (np.array(bits, np.float64) * angle).astype(np.float32).reshape(1, L, 1, 1)
    d = {"x": x, "B": e0, "C": e0.copy(), "dt": np.ones((1, L, 1), np.float32),
         "lam": np.ones((1, L, 1), np.float32), "theta": th,
         "A_log": np.array([-np.inf], np.float32), "B_bias": None, "C_bias": None, "init": None}
    return ref.scan_seq(d)[0][0, :, 0, 0, 0]


def test_parity_and_mod5():
    """[M3] "Why a rotating state can count": a turn of pi per 1 flips a fixed
    readout of the first coordinate on every 1 (parity); a turn of 2 pi / 5
    returns to the start after five 1s and not before (counting mod 5)."""
    bits = [1, 1, 0, 1, 1, 1, 0, 0, 1, 0, 1, 1, 1, 1, 0, 1]
    y = _counter(bits, math.pi)
    ones = np.cumsum(bits) - bits[0]                # ones after the write at t = 0
    np.testing.assert_allclose(y, (-1.0) ** ones, atol=1e-6)
    y5 = _counter([1] * 16, 2 * math.pi / 5)
    k = np.arange(16)
    back = np.isclose(y5, 1.0, atol=1e-6)
    assert np.array_equal(back, k % 5 == 0)


# --------------------------------------------------------------------------
# pin 8: MIMO = sum of SISO problems
# --------------------------------------------------------------------------
def test_mimo_decomposition():
    """[M3] "MIMO": R writes share one decay, are summed into one state and read
    R times, so readout r is the sum over writes r' of SISO runs with
    (x_r', B_r', C_r); R identical ranks give R times the SISO output."""
    cfg, d = make_small_case(31, batch=1, seqlen=11, nheads=1, headdim=3, dstate=6,
                             rank=3, npairs=2, bias=True, init_full=False)
    y, _ = ref.scan_seq(d)
    Bb = d["B"].astype(np.float64) + d["B_bias"][None, None].astype(np.float64)
    Cb = d["C"].astype(np.float64) + d["C_bias"][None, None].astype(np.float64)
    for r in range(3):
        acc = 0.0
        for q in range(3):
            s = dict(d, x=d["x"][:, :, :, q:q + 1], B=Bb[:, :, :, q:q + 1], C=Cb[:, :, :, r:r + 1],
                     B_bias=None, C_bias=None)
            acc = acc + ref.scan_seq(s)[0][:, :, :, 0]
        assert _rel(y[:, :, :, r], acc) < 1e-12
    same = dict(d, x=np.repeat(d["x"][:, :, :, :1], 3, axis=3), B=np.repeat(d["B"][:, :, :, :1], 3, axis=3),
                C=np.repeat(d["C"][:, :, :, :1], 3, axis=3), B_bias=None, C_bias=None)
    ys, _ = ref.scan_seq(same)
    y1, _ = ref.scan_seq(dict(same, x=same["x"][:, :, :, :1], B=same["B"][:, :, :, :1],
                              C=same["C"][:, :, :, :1]))
    for r in range(3):
        assert _rel(ys[:, :, :, r], 3.0 * y1[:, :, :, 0]) < 1e-12


# --------------------------------------------------------------------------
# pin 9: continuation -- whole = split = token by token
# --------------------------------------------------------------------------
def _slice(d, t0, t1, init):
    out = dict(d)
    for k in ("x", "B", "C", "dt", "lam", "theta"):
        if d.get(k) is not None:
            out[k] = d[k][:, t0:t1]
    out["init"] = init
    return out


@pytest.mark.parametrize("split", [1, 5, 9])
def test_continuation(split):
    """[D] Appendix C.2: initial and final carries (state, phase, previous
    write) make whole-sequence, split-sequence and token-by-token evaluation
    agree.  [M3] decode listing: the decode step is one token with the carry."""
    _, d = make_small_case(41, batch=2, seqlen=12, nheads=2, ngroups=1, headdim=3,
                           dstate=6, rank=2, npairs=2, init_full=True)
    y, f = ref.scan_seq(d)
    ya, fa = ref.scan_seq(_slice(d, 0, split, d["init"]))
    yb, fb = ref.scan_seq(_slice(d, split, 12, fa))
    assert _rel(np.concatenate([ya, yb], axis=1), y) < 1e-12
    for k in ("h", "B_prev", "x_prev"):
        assert _rel(fb[k], f[k]) < 1e-12
    assert np.allclose(np.cos(fb["phi"]), np.cos(f["phi"]), atol=1e-12)
    carry = {k: np.asarray(v, np.float64) for k, v in d["init"].items()}
    ys = []
    for t in range(12):
        yt, carry = ref.decode_step(carry, d["x"][:, t], d["B"][:, t], d["C"][:, t], d["dt"][:, t],
                                    d["lam"][:, t], d["theta"][:, t], d["A_log"], d["B_bias"], d["C_bias"])
        ys.append(yt)
    assert _rel(np.stack(ys, axis=1), y) < 1e-12
    assert _rel(carry["h"], f["h"]) < 1e-12


# --------------------------------------------------------------------------
# pin 10: shared groups + per-head bias = materialised per-head B, C
# --------------------------------------------------------------------------
def test_group_bias_reduction():
    """[M3] "MIMO" (B and C shared across the heads of a layer) and "The Mamba-3
    block" (a per-head bias on B and C): G = 1 plus a bias equals per-head
    tensors B + b_h, C + c_h with G = H and no bias."""
    _, d = make_small_case(51, batch=2, seqlen=9, nheads=3, ngroups=1, headdim=3,
                           dstate=6, rank=2, npairs=2, bias=True, init_full=True)
    y, f = ref.scan_seq(d)
    Bh = d["B"].astype(np.float64) + d["B_bias"][None, None]   # [b,L,H,R,N]: G=1 broadcast over H
    Ch = d["C"].astype(np.float64) + d["C_bias"][None, None]
    e = dict(d, B=Bh.astype(np.float64), C=Ch.astype(np.float64), B_bias=None, C_bias=None)
    y2, f2 = ref.scan_seq(e)
    assert _rel(y2, y) < 1e-12 and _rel(f2["h"], f["h"]) < 1e-12
    y3, _ = ref_cpu.scan(dict(e, B=Bh.astype(np.float32), C=Ch.astype(np.float32)))
    assert _rel(y3, y) < 1e-6        # the float32 rounding of B + bias only


# --------------------------------------------------------------------------
# pin 11: superposition in (carry, input)
# --------------------------------------------------------------------------
def test_superposition():
    """[D] Section 1 ("including the initial-state contribution") and the
    linearity of the recurrence in the state: y(carry, x) = y(carry, 0) +
    y(0, x) with the phase carry held fixed."""
    _, d = make_small_case(61, batch=1, seqlen=10, nheads=2, headdim=3, dstate=6,
                           rank=2, npairs=3, init_full=True)
    y, f = ref.scan_seq(d)
    z = dict(d, x=np.zeros_like(d["x"]))
    zi = dict(d["init"], h=np.zeros_like(d["init"]["h"]), B_prev=np.zeros_like(d["init"]["B_prev"]),
              x_prev=np.zeros_like(d["init"]["x_prev"]))
    yc, fc = ref.scan_seq(z)
    yx, fx = ref.scan_seq(dict(d, init=zi))
    assert _rel(yc + yx, y) < 1e-12
    assert _rel(fc["h"] + fx["h"], f["h"]) < 1e-12


# --------------------------------------------------------------------------
# pin 12: the pages' byte and operation counts of a decode step
# --------------------------------------------------------------------------
def test_byte_and_op_model():
    """[M3] "Why a recurrent model's decode step is memory-bound" (17,026 bytes,
    5NP - P = 40,896 ops, intensity 2.4) and "MIMO" (18,946 bytes, 4NPR + NP -
    PR = 139,008 ops, ratio 3.40; full round trip about 1.2 and 3.9)."""
    assert model.decode_bytes_paper(64, 128, 1) == 17026
    assert model.decode_bytes_paper(64, 128, 4) == 18946
    assert model.decode_ops_paper(64, 128, 1) == 40896 == 5 * 128 * 64 - 64
    assert model.decode_ops_paper(64, 128, 4) == 139008
    assert round(model.intensity(40896, 17026), 1) == 2.4
    assert round(139008 / 40896, 2) == 3.40
    assert round(model.intensity(40896, model.decode_bytes_round_trip(64, 128, 1)), 1) == 1.2
    assert round(model.intensity(139008, model.decode_bytes_round_trip(64, 128, 4)), 1) == 3.9


@pytest.mark.parametrize("P,N,R", [(64, 128, 1), (64, 128, 4), (3, 5, 2), (2, 7, 3)])
def test_counted_decode_step(P, N, R):
    """An instrumented decode step (lam = 1, no rotation) performs exactly
    5NP - P (R = 1) or 4NPR + NP - PR operations, and computes the same
    values as the oracle's decode step."""
    rng = np.random.default_rng(P * 1000 + N * 10 + R)
    h = rng.standard_normal((P, N))
    x = rng.standard_normal((R, P))
    B = rng.standard_normal((R, N))
    C = rng.standard_normal((R, N))
    dt, A_log = 0.3, 0.2
    alpha = math.exp(-dt * math.exp(A_log))
    hn, y, nops = ref.counted_decode_step(h.tolist(), x.tolist(), B.tolist(), C.tolist(), alpha, dt)
    if R == 1:
        assert nops == 5 * N * P - P
    assert nops == 4 * N * P * R + N * P - P * R == model.decode_ops_paper(P, N, R)
    carry = {"h": h[None, None], "phi": np.zeros((1, 1, 0)), "B_prev": np.zeros((1, 1, R, N)),
             "x_prev": np.zeros((1, 1, R, P))}
    y2, c2 = ref.decode_step(carry, x[None, None], B[None, None], C[None, None], np.full((1, 1), dt),
                             np.ones((1, 1)), None, np.array([A_log]))
    assert _rel(np.array(y), y2[0, 0]) < 1e-12
    assert _rel(np.array(hn), c2["h"][0, 0]) < 1e-12


# --------------------------------------------------------------------------
# pin 14: per-token decay rates (the heavy-tail law)
# --------------------------------------------------------------------------
def test_heavy_tail_rate_closed_form():
    """[M3] remarks after the decode listing: heavy_tail(u) is 1 + u for
    u >= 0 and 1 / (1 - u) for u < 0; the rate is its negation clamped at
    -1e-4.  Values by hand, the floor, and the joint at u = 0 (value and slope
    1 from both sides)."""
    u = np.array([0.0, 2.0, 0.5, -1.0, -3.0, -1e5, -1e9, 7.0])
    want = np.array([-1.0, -3.0, -1.5, -0.5, -0.25, -1e-4, -1e-4, -8.0])
    assert np.array_equal(ref.heavy_tail_rate(u), want)
    assert float(ref.heavy_tail_rate(-9998.0)) == pytest.approx(-1.0 / 9999.0, rel=1e-15)  # just above the floor
    e = 1e-7
    left = (ref.heavy_tail_rate(0.0) - ref.heavy_tail_rate(-e)) / e
    right = (ref.heavy_tail_rate(e) - ref.heavy_tail_rate(0.0)) / e
    assert left == pytest.approx(-1.0, abs=1e-6) and right == pytest.approx(-1.0, abs=1e-6)
    grid = np.linspace(-50.0, 50.0, 2001)
    assert np.all(np.diff(ref.heavy_tail_rate(grid)) < 0)      # strictly decreasing above the floor


def _case_scalar_dyn(dts, lams, xs, us):
    d = _case_scalar(dts, lams, xs)
    d["A_raw"] = np.array(us, np.float32).reshape(1, len(xs), 1)
    d["A_log"] = np.array([123.0], np.float32)       # must not be read
    return d


@pytest.mark.parametrize("form", sorted(ALL_FORMS))
def test_dynamic_rate_worked_example(form):
    """[M3] worked step with the rate input u = 0 (heavy_tail = 1, A = -1)
    reproduces the page's 0.35, 0.303, 0.184; with u = (0, 1, -1) token t's
    own rate decays the state entering token t: 0.35, e^{-1} 0.5 and
    e^{-1/4} e^{-1} 0.5 by hand."""
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    fn = ALL_FORMS[form]
    y, _ = fn(_case_scalar_dyn([0.5] * 3, [0.7] * 3, [1.0, 0.0, 0.0], [0.0, 0.0, 0.0]))
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    np.testing.assert_allclose(y.reshape(-1), g["mamba3_states"], atol=tol)
    y, _ = fn(_case_scalar_dyn([0.5] * 3, [0.7] * 3, [1.0, 0.0, 0.0], [0.0, 1.0, -1.0]))
    h1 = math.exp(0.5 * -2.0) * 0.5          # a_1 (gamma_0 + delta_1) x_0, A_1 = -2
    h2 = math.exp(0.5 * -0.5) * h1           # A_2 = -1/2
    assert np.allclose(y.reshape(-1), [0.35, h1, h2], rtol=1e-6, atol=0)


def test_dynamic_rate_equals_static():
    """A per-token rate input that is constant per head, u = exp(A_log) - 1
    (heavy_tail(u) = exp(A_log) on the u >= 0 branch), gives the static-rate
    result; and so does u = 1 - exp(-A_log) on the u < 0 branch for heads
    whose rate magnitude is below 1."""
    _, d = make_small_case(131, batch=2, seqlen=14, nheads=3, ngroups=1, headdim=3, dstate=6, rank=2,
                           npairs=2, init_full=True, dt_scale=2.0)
    d["A_log"] = np.array([0.3, 1.7, -0.9])          # exp: 1.35, 5.47, 0.41
    y0, f0 = ref.scan_seq(d)
    a = np.exp(d["A_log"])
    u = np.where(a >= 1.0, a - 1.0, 1.0 - 1.0 / a)
    dd = dict(d, A_raw=np.broadcast_to(u, (2, 14, 3)).copy(), A_log=None)
    for fn in (ref.scan_seq, ref.scan_quadratic, lambda z: ref.scan_chunked(z, 4), ref.scan_seq_unrotated):
        y1, f1 = fn(dd)
        assert _rel(y1, y0) < 1e-12
        assert _rel(f1["h"], f0["h"]) < 1e-12


@pytest.mark.parametrize("seed,R,npairs,L", [(141, 1, 0, 11), (142, 3, 2, 13), (143, 4, 3, 10)])
def test_dynamic_rate_forms_agree(seed, R, npairs, L):
    """With rates that change every token (u ~ N(0, 4), both branches and some
    at the floor): the explicit decay products of the masked form, the
    sequential recurrence, the chunk-local log-sums at every chunk size, the
    unrotated state and the C recurrence all agree."""
    _, d = make_small_case(seed, batch=2, seqlen=L, nheads=2, ngroups=1, headdim=3, dstate=6, rank=R,
                           npairs=npairs, init_full=True, dt_scale=2.0, rate_dyn=True)
    d["A_raw"] = (d["A_raw"] * 2.0).astype(np.float32)
    d["A_raw"][0, 1, 0] = -2e4                        # one floored token
    y0, f0 = ref.scan_seq(d)
    yq, fq = ref.scan_quadratic(d)
    assert _rel(yq, y0) < 1e-12 and _rel(fq["h"], f0["h"]) < 1e-12
    for q in range(1, L + 1):
        yc, fc = ref.scan_chunked(d, q)
        assert _rel(yc, y0) < 1e-12 and _rel(fc["h"], f0["h"]) < 1e-12, q
    yu, fu = ref.scan_seq_unrotated(d)
    assert _rel(yu, y0) < 1e-12
    yc, fc = ref_cpu.scan(d)
    assert _rel(yc, y0) < 1e-12 and _rel(fc["h"], f0["h"]) < 1e-12
    # a rate that differs from the static one changes the result
    ys, _ = ref.scan_seq(dict(d, A_raw=None))
    assert _rel(ys, y0) > 1e-2


def test_dynamic_rate_decode_continuation():
    """[M3] decode listing (A = -heavy_tail(A_r) per token): token-by-token
    decode with per-token rate inputs equals the whole-sequence scan."""
    _, d = make_small_case(151, batch=2, seqlen=9, nheads=2, ngroups=1, headdim=3, dstate=6, rank=2,
                           npairs=2, init_full=True, rate_dyn=True)
    y, f = ref.scan_seq(d)
    carry = {k: np.asarray(v, np.float64) for k, v in d["init"].items()}
    ys = []
    for t in range(9):
        yt, carry = ref.decode_step(carry, d["x"][:, t], d["B"][:, t], d["C"][:, t], d["dt"][:, t],
                                    d["lam"][:, t], d["theta"][:, t], None, d["B_bias"], d["C_bias"],
                                    A_raw=d["A_raw"][:, t])
        ys.append(yt)
    assert _rel(np.stack(ys, axis=1), y) < 1e-12
    assert _rel(carry["h"], f["h"]) < 1e-12


# --------------------------------------------------------------------------
# the C oracle against the numpy oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed,G,R,npairs,bias", [
    (71, 1, 4, 3, True), (72, 2, 1, 0, False), (73, 4, 2, 4, True), (74, 1, 3, 1, False)])
def test_c_oracle_matches_numpy(seed, G, R, npairs, bias):
    """The plain-C recurrence and the numpy recurrence agree to 1e-12 on
    random cases with groups, bias, full carries and selected streams."""
    _, d = make_small_case(seed, batch=2, seqlen=19, nheads=4, ngroups=G, headdim=5,
                           dstate=8, rank=R, npairs=npairs, bias=bias, init_full=True)
    y0, f0 = ref.scan_seq(d)
    y1, f1 = ref_cpu.scan(d)
    assert _rel(y1, y0) < 1e-12
    for k in ("h", "B_prev", "x_prev", "phi"):
        assert _rel(f1[k], f0[k]) < 1e-12, k
    sel = [(1, 3), (0, 2)]
    ys, fs = ref_cpu.scan(d, sel=sel)
    for i, (bi, h) in enumerate(sel):
        assert _rel(ys[i], y0[bi, :, h]) < 1e-12
        assert _rel(fs["h"][i], f0["h"][bi, h]) < 1e-12


def test_c_oracle_rejects_bad_arguments():
    _, d = make_small_case(81, nheads=3, ngroups=2)
    with pytest.raises(RuntimeError):
        ref_cpu.scan(d)


# --------------------------------------------------------------------------
# planted mistakes: each plausible slip in the oracle fails some pin above
# --------------------------------------------------------------------------
def test_planted_mistakes_are_caught(monkeypatch):
    """Plant, on the CPU, the slips a from-scratch implementation is likely to
    make, and check that the independent pins catch each one."""
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    # (a) lagged term weighted by the earlier token's lam: breaks the lam = 0.2 case
    s = _case_scalar([0.5] * 3, [0.7, 0.2, 0.7], [1.0, 0.0, 0.0])
    e = math.exp(-0.5)
    wrong_second = e * 0.35 + e * 0.5 * (1 - 0.7)          # uses lam_1 instead of lam_2
    assert abs(wrong_second - g["second_token_lam_0p2"]["state_after_second"]) > 0.05
    y, _ = ref.scan_seq(s)
    assert abs(y.reshape(-1)[1] - g["second_token_lam_0p2"]["state_after_second"]) < 5e-4
    # (b) rotation turned the other way for C only: breaks the rotated/unrotated pin
    orig = ref.rot
    _, d = make_small_case(21, batch=1, seqlen=8, nheads=1, headdim=2, dstate=4, rank=1, npairs=2,
                           init_full=False)
    d["theta"] = (d["theta"] * 300.0).astype(np.float32)
    y_ok, _ = ref.scan_seq(d)
    calls = {"n": 0}

    def bad_rot(v, phi):
        calls["n"] += 1
        return orig(v, -phi if calls["n"] % 2 == 0 else phi)   # every second call (C) flips
    monkeypatch.setattr(ref, "rot", bad_rot)
    y_bad, _ = ref.scan_seq(d)
    monkeypatch.setattr(ref, "rot", orig)
    assert _rel(y_bad, y_ok) > 1e-3
    # (d) the decay of token t taken from token t - 1's rate input: breaks the
    # per-token worked example (0.303 instead of e^{-1} 0.5 = 0.184)
    orig_rate = ref._rate_mag

    def lagged_rate(inp, bi, h, L):
        a = orig_rate(inp, bi, h, L)
        return np.concatenate([a[:1], a[:-1]])
    dd = _case_scalar_dyn([0.5] * 3, [0.7] * 3, [1.0, 0.0, 0.0], [0.0, 1.0, -1.0])
    monkeypatch.setattr(ref, "_rate_mag", lagged_rate)
    y_bad, _ = ref.scan_seq(dd)
    monkeypatch.setattr(ref, "_rate_mag", orig_rate)
    assert abs(y_bad.reshape(-1)[1] - math.exp(-1.0) * 0.5) > 0.1
    # (c) a dropped lagged term: breaks the worked example
    s2 = _case_scalar([0.5] * 3, [0.7] * 3, [1.0, 0.0, 0.0])
    y2, _ = ref.scan_seq(s2)
    assert abs(y2.reshape(-1)[1] - e * 0.35) > 0.05   # without the lag it would read 0.212
