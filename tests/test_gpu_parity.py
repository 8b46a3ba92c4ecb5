"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (normwise relative L2 per tensor): 1e-4 for f32 I/O, 2e-2 for
bf16 I/O, as the workload statement fixes.  Phases are compared through
(cos, sin) with an absolute bound.
"""
import sys

import numpy as np
import pytest

from m3inputs import CONFIGS, config_by_name, make_decode_inputs, make_scan_inputs, make_small_case
from oracle import ref_cpu
from tests._util import ROW_TOL, host, phase_err, pooled_signed, rel_l2, row_errors, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def m3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_mimo_amd as m
    return m


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tol(io):
    return 1e-4 if io == "f32" else 2e-2


def _run_scan(m3, d, cfg, chunk=None, nsegments=0):
    dev = torch.device("cuda:0")
    io = torch.float32 if cfg.io_dtype == "f32" else torch.bfloat16
    sd = torch.float32 if cfg.state_dtype == "f32" else torch.bfloat16
    t = to_device(d, io, sd, dev)
    y, fin = m3.scan_fwd(t["x"], t["B"], t["C"], t["dt"], t["lam"], t["theta"], t["A_log"], t["B_bias"],
                         t["C_bias"], t["init"], chunk=chunk or cfg.chunk, state_dtype=sd, nsegments=nsegments,
                         A_raw=t["A_raw"])
    torch.cuda.synchronize()
    return y, fin


def _compare(y, fin, yr, fr, io, sel=None, what=""):
    tol = _tol(io)
    yg = host(y)
    if sel is not None:
        yg = np.stack([yg[bi, :, h] for bi, h in sel])
    e = rel_l2(yg, yr)
    bias = pooled_signed(yg, yr)
    _say("  %s y rel-L2 %.3e  pooled-signed %.2e" % (what, e, bias))
    assert e <= tol, "y rel-L2 %.3e > %.1e" % (e, tol)
    assert abs(bias) <= tol / 4
    if fin is None:
        return
    for k in ("h", "B_prev", "x_prev"):
        g = host(fin[k])
        if sel is not None:
            g = np.stack([g[bi, h] for bi, h in sel])
        ek = rel_l2(g, fr[k])
        _say("  %s %s rel-L2 %.3e" % (what, k, ek))
        assert ek <= tol, k
    if fr["phi"].size:
        g = host(fin["phi"])
        if sel is not None:
            g = np.stack([g[bi, h] for bi, h in sel])
        assert phase_err(g, fr["phi"]) < 1e-3
        assert g.min() >= 0.0 and g.max() < 2 * np.pi + 1e-6


# -----------------------------------------------------------------------------
# small feature sweep (oracle on every stream)
# -----------------------------------------------------------------------------
SWEEP = [
    # io,   P,  N, R, np, G, Q, L,  bias, lam1, init
    ("f32", 16, 16, 1, 4, 2, 16, 64, False, False, False),
    ("f32", 16, 16, 2, 8, 1, 16, 37, True, False, True),
    ("f32", 8, 12, 3, 0, 1, 5, 23, True, True, True),
    ("f32", 64, 128, 4, 32, 1, 64, 70, True, False, True),
    ("f32", 64, 128, 1, 0, 1, 64, 129, False, True, False),
    ("bf16", 16, 16, 1, 4, 2, 16, 64, False, False, False),
    ("bf16", 64, 128, 1, 0, 1, 64, 130, False, True, False),
    ("bf16", 64, 128, 2, 32, 1, 32, 100, True, False, True),
    ("bf16", 64, 128, 4, 32, 1, 64, 150, True, False, True),
    ("bf16", 64, 128, 4, 64, 2, 16, 77, True, False, True),
    ("bf16", 64, 128, 4, 0, 1, 128, 300, True, False, True),
    ("bf16", 32, 64, 2, 8, 1, 32, 64, False, False, True),
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: "%s-P%d-N%d-R%d-np%d-G%d-Q%d-L%d" % c[:8])
def test_scan_sweep(m3, case):
    io, P, N, R, npairs, G, Q, L, bias, lam1, init = case
    _say("scan sweep", case)
    cfg, d = make_small_case(1000 + P + N + R + Q + L, batch=2, seqlen=L, nheads=4, ngroups=G, headdim=P,
                             dstate=N, rank=R, npairs=npairs, chunk=Q, io_dtype=io, state_dtype="f32",
                             bias=bias, lam_one=lam1, rms_bc=(io == "bf16"), init_full=init)
    yr, fr = ref_cpu.scan(d)
    y, fin = _run_scan(m3, d, cfg)
    _compare(y, fin, yr, fr, io, what="sweep")


# bf16, P = 64, N = 128: the MFMA route, every (R, Q) specialisation, one
# sequence segment and several (the segmented schedule), ragged lengths.
MFMA = [
    # R, Q,   np, G, L,   bias, lam1, init, nseg
    (1, 64, 0, 1, 130, False, True, False, 1),
    (1, 64, 32, 1, 200, True, False, True, 3),
    (1, 128, 16, 2, 300, True, False, True, 1),
    (2, 32, 32, 1, 100, True, False, True, 1),
    (2, 32, 8, 1, 161, True, False, True, 4),
    (2, 64, 32, 1, 129, True, False, True, 2),
    (2, 128, 32, 2, 260, False, False, True, 1),
    (4, 16, 64, 2, 77, True, False, True, 1),
    (4, 16, 32, 1, 96, True, False, True, 6),
    (4, 32, 32, 1, 99, True, False, True, 2),
    (4, 64, 32, 1, 150, True, False, True, 1),
    (4, 64, 32, 1, 250, True, False, True, 3),
    (4, 64, 0, 1, 64, True, True, False, 1),
    (4, 128, 32, 1, 300, True, False, True, 1),
    (4, 128, 32, 1, 520, True, False, True, 4),
    # every pair turning at the longest chunk (the largest angle staging)
    (4, 128, 64, 1, 200, True, False, True, 2),
    (1, 128, 64, 2, 150, True, False, True, 1),
]


@pytest.mark.parametrize("case", MFMA, ids=lambda c: "R%d-Q%d-np%d-G%d-L%d-seg%d" % (c[:5] + c[8:]))
def test_scan_mfma(m3, case):
    R, Q, npairs, G, L, bias, lam1, init, nseg = case
    _say("mfma scan", case)
    cfg, d = make_small_case(2000 + 7 * R + Q + L + nseg, batch=2, seqlen=L, nheads=4, ngroups=G, headdim=64,
                             dstate=128, rank=R, npairs=npairs, chunk=Q, io_dtype="bf16", state_dtype="f32",
                             bias=bias, lam_one=lam1, rms_bc=True, init_full=init)
    yr, fr = ref_cpu.scan(d)
    y, fin = _run_scan(m3, d, cfg, nsegments=nseg)
    _compare(y, fin, yr, fr, "bf16", what="mfma")


# The single-rank path without rotation or bias (head-shared scores per batch, group and
# chunk, then the scan per batch, head and half of P): the trapezoid term and the carries,
# groups, ragged and short sequences, per-token rates; every output row bounded on its own.
SISO = [
    # L,   G, H, lam1,  init,  dyn
    (130, 1, 4, True, False, False),
    (200, 1, 4, False, True, False),
    (64, 2, 4, False, True, False),
    (1, 1, 2, False, True, False),
    (37, 1, 3, False, False, False),
    (300, 2, 4, False, True, True),
    (2048, 1, 2, False, True, False),
]


@pytest.mark.parametrize("case", SISO, ids=lambda c: "L%d-G%d-H%d-lam1%d-init%d-dyn%d" % c)
def test_scan_siso(m3, case):
    L, G, H, lam1, init, dyn = case
    _say("siso scan", case)
    cfg, d = make_small_case(5000 + L + 7 * G + H + 3 * init + dyn, batch=2, seqlen=L, nheads=H, ngroups=G, headdim=64,
                             dstate=128, rank=1, npairs=0, chunk=64, io_dtype="bf16", state_dtype="f32",
                             bias=False, lam_one=lam1, rms_bc=True, init_full=init, rate_dyn=dyn)
    yr, fr = ref_cpu.scan(d)
    y, fin = _run_scan(m3, d, cfg)
    _compare(y, fin, yr, fr, "bf16", what="siso")
    er = float(row_errors(host(y), np.asarray(yr)).max())
    _say("  siso worst row %.3e" % er)
    assert er <= ROW_TOL


def test_scan_segments_agree(m3):
    """The schedule (number of segments) changes rounding only."""
    cfg, d = make_small_case(3003, batch=1, seqlen=512, nheads=2, ngroups=1, headdim=64, dstate=128, rank=4,
                             npairs=32, chunk=64, io_dtype="bf16", rms_bc=True, init_full=True)
    yr, fr = ref_cpu.scan(d)
    ys = []
    for k in (1, 2, 4, 8):
        y, fin = _run_scan(m3, d, cfg, nsegments=k)
        _compare(y, fin, yr, fr, "bf16", what="nseg=%d" % k)
        ys.append(host(y))
    for yk in ys[1:]:
        assert rel_l2(yk, ys[0]) < 1e-2


@pytest.mark.parametrize("nseg", [16, 33, 100])
def test_scan_many_segments(m3, nseg):
    """More segments than one lane group of the carry scan holds: 16 (one group of 16
    lanes), 33 (one 64-lane block, partly filled) and 100 (two blocks of 64, the second
    entered with the first's carried state and angle), each against the oracle."""
    cfg, d = make_small_case(3031 + nseg, batch=1, seqlen=2000, nheads=2, ngroups=1, headdim=64, dstate=128, rank=4,
                             npairs=32, chunk=16, io_dtype="bf16", rms_bc=True, init_full=True)
    yr, fr = ref_cpu.scan(d)
    y, fin = _run_scan(m3, d, cfg, nsegments=nseg)
    _compare(y, fin, yr, fr, "bf16", what="nseg=%d" % nseg)


def test_long_chunk_request_is_split(m3):
    """A chunk longer than the matrix-core path's 256 rows (R = 4, Q = 128) runs
    on the small-chunk schedule (16 tokens): the same schedule, hence the same
    bits, as asking for 16."""
    cfg, d = make_small_case(3011, batch=2, seqlen=300, nheads=2, ngroups=1, headdim=64, dstate=128, rank=4,
                             npairs=32, chunk=128, io_dtype="bf16", rms_bc=True, init_full=True)
    y128, f128 = _run_scan(m3, d, cfg, chunk=128)
    y16, f16 = _run_scan(m3, d, cfg, chunk=16)
    assert torch.equal(y128, y16) and torch.equal(f128["h"], f16["h"])
    yr, fr = ref_cpu.scan(d)
    _compare(y128, f128, yr, fr, "bf16", what="Q128 -> 16")


def test_config1_tiny_siso_f32(m3):
    cfg = config_by_name("tiny_siso_f32")
    d = make_scan_inputs(cfg)
    yr, fr = ref_cpu.scan(d)
    y, fin = _run_scan(m3, d, cfg)
    _compare(y, fin, yr, fr, cfg.io_dtype, what="config1")


def test_scan_empty_sequence(m3):
    """L = 0: nothing but the carry copy (zeros without an initial carry)."""
    cfg, d = make_small_case(5, batch=2, seqlen=0, nheads=2, headdim=8, dstate=8, rank=2, npairs=2,
                             init_full=True)
    y, fin = _run_scan(m3, d, cfg)
    assert y.numel() == 0
    for k in ("h", "phi", "B_prev", "x_prev"):
        np.testing.assert_array_equal(host(fin[k]), d["init"][k].astype(np.float64))
    d["init"] = None
    y, fin = _run_scan(m3, d, cfg)
    for k in ("h", "phi", "B_prev", "x_prev"):
        assert not host(fin[k]).any()


def test_scan_deterministic(m3):
    cfg, d = make_small_case(7, batch=2, seqlen=150, nheads=4, ngroups=1, headdim=64, dstate=128, rank=4,
                             npairs=32, chunk=64, io_dtype="bf16", rms_bc=True, init_full=True)
    y1, f1 = _run_scan(m3, d, cfg)
    y2, f2 = _run_scan(m3, d, cfg)
    assert torch.equal(y1, y2) and torch.equal(f1["h"], f2["h"])


# per-token (heavy-tail) decay rates: the generic route (f32), the MFMA route
# (bf16, one and several segments) and the decode step
RATE_DYN = [
    # io,   P,  N,   R, np, G, Q,  L,   nseg
    ("f32", 16, 16, 2, 4, 1, 16, 45, 0),
    ("f32", 64, 128, 4, 32, 1, 64, 70, 0),
    ("bf16", 64, 128, 4, 32, 1, 64, 150, 1),
    ("bf16", 64, 128, 4, 32, 1, 64, 250, 3),
    ("bf16", 64, 128, 1, 0, 2, 128, 200, 1),
    ("bf16", 64, 128, 2, 16, 1, 32, 161, 2),
    ("bf16", 64, 128, 4, 32, 1, 16, 90, 2),
]


@pytest.mark.parametrize("case", RATE_DYN, ids=lambda c: "%s-P%d-N%d-R%d-np%d-G%d-Q%d-L%d-seg%d" % c)
def test_scan_dynamic_rate(m3, case):
    """Per-token rates A_t = min(-heavy_tail(u_t), -1e-4) (M3_RATE_HEAVY_TAIL);
    u ~ N(0, 1) spans both branches of the law."""
    io, P, N, R, npairs, G, Q, L, nseg = case
    _say("dynamic-rate scan", case)
    cfg, d = make_small_case(4000 + P + R + Q + L + nseg, batch=2, seqlen=L, nheads=4, ngroups=G, headdim=P,
                             dstate=N, rank=R, npairs=npairs, chunk=Q, io_dtype=io, state_dtype="f32",
                             bias=True, rms_bc=(io == "bf16"), init_full=True, rate_dyn=True)
    yr, fr = ref_cpu.scan(d)
    y, fin = _run_scan(m3, d, cfg, nsegments=nseg)
    _compare(y, fin, yr, fr, io, what="dyn-rate")


@pytest.mark.parametrize("Q", [16, 64])
@pytest.mark.parametrize("dt_scale", [40.0, 1e-3])
def test_scan_extreme_decay(m3, Q, dt_scale):
    """Steps 40x the workload law (per-token log-decays down to about -1e3, so a
    chunk's decay underflows fp32) and 1e-3x (decays within 1e-3 of one): the
    weights are exps of non-positive log-decay differences, so neither end
    overflows or loses the diagonal terms."""
    cfg, d = make_small_case(4200 + Q, batch=2, seqlen=150, nheads=2, ngroups=1, headdim=64, dstate=128, rank=4,
                             npairs=32, chunk=Q, io_dtype="bf16", rms_bc=True, init_full=True, dt_scale=dt_scale)
    yr, fr = ref_cpu.scan(d)
    y, fin = _run_scan(m3, d, cfg)
    assert torch.isfinite(y.float()).all() and torch.isfinite(fin["h"]).all()
    _compare(y, fin, yr, fr, "bf16", what="dt x %g" % dt_scale)


def test_scan_dynamic_rate_floor(m3):
    """Very negative rate inputs hit the -1e-4 floor: long memory, through the
    MFMA route, against the oracle."""
    cfg, d = make_small_case(4100, batch=1, seqlen=200, nheads=2, ngroups=1, headdim=64, dstate=128, rank=4,
                             npairs=32, chunk=64, io_dtype="bf16", rms_bc=True, init_full=True, rate_dyn=True)
    d["A_raw"][:, ::2] = np.float32(-3e4)      # |A| = 1/(1 + 3e4) < 1e-4: floored
    yr, fr = ref_cpu.scan(d)
    y, fin = _run_scan(m3, d, cfg)
    _compare(y, fin, yr, fr, "bf16", what="dyn-rate floor")


# -----------------------------------------------------------------------------
# decode step
# -----------------------------------------------------------------------------
DECODE = [
    # io,   state, P,  N,  R, np, G, steps
    ("f32", "f32", 16, 16, 1, 4, 2, 5),
    ("bf16", "bf16", 64, 128, 4, 32, 1, 12),
    ("bf16", "bf16", 64, 128, 2, 16, 2, 6),
    ("bf16", "bf16", 64, 128, 1, 0, 1, 6),
    ("bf16", "f32", 64, 128, 4, 32, 1, 5),
    ("bf16", "bf16", 32, 64, 4, 8, 1, 5),
    # per-token (heavy-tail) rates
    ("f32", "f32", 16, 16, 2, 4, 1, 5, True),
    ("bf16", "f32", 64, 128, 4, 32, 1, 6, True),
]


@pytest.mark.parametrize("case", DECODE, ids=lambda c: "%s-%s-P%d-N%d-R%d-np%d-G%d-S%d" % c[:8]
                         + ("-dyn" if len(c) > 8 else ""))
def test_decode_steps(m3, case):
    """k decode steps through m3_decode_step equal the oracle's recurrence over
    k tokens (carried state, phase, previous write)."""
    io, sdt, P, N, R, npairs, G, steps = case[:8]
    dyn = len(case) > 8 and case[8]
    _say("decode", case)
    cfg, _ = make_small_case(0, batch=3, seqlen=steps, nheads=4, ngroups=G, headdim=P, dstate=N, rank=R,
                             npairs=npairs, io_dtype=io, state_dtype=sdt, bias=True, rms_bc=(io == "bf16"),
                             rate_dyn=dyn)
    cfg = cfg.with_(init_state=True, init_full=True)
    d = make_decode_inputs(cfg, steps, seed=77)
    yr, fr = ref_cpu.scan(d)
    dev = torch.device("cuda:0")
    iot = torch.float32 if io == "f32" else torch.bfloat16
    sdt_t = torch.float32 if sdt == "f32" else torch.bfloat16
    t = to_device(d, iot, sdt_t, dev)
    carry = {k: v.clone() for k, v in t["init"].items()}
    ys = []
    for s in range(steps):
        ys.append(m3.decode_step(t["x"][:, s].contiguous(), t["B"][:, s].contiguous(), t["C"][:, s].contiguous(),
                                 t["dt"][:, s].contiguous(), t["lam"][:, s].contiguous(),
                                 None if t["theta"] is None else t["theta"][:, s].contiguous(),
                                 t["A_log"], t["B_bias"], t["C_bias"], carry,
                                 A_raw=None if t["A_raw"] is None else t["A_raw"][:, s].contiguous()))
    torch.cuda.synchronize()
    y = torch.stack(ys, dim=1)
    _compare(y, carry, yr, fr, io, what="decode")
