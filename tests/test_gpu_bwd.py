"""GPU parity of the scan's backward pass (``m3_scan_bwd`` through the C ABI)
against the fp64 backward oracle (``oracle.grad``), every gradient tensor.

Tolerances (normwise relative L2 per tensor): 1e-4 for f32 I/O, 2e-2 for bf16
I/O (inputs and dy rounded to bf16 on both sides; the kernels accumulate in
fp32 and round dx, dB, dC to bf16).
"""
import sys

import numpy as np
import pytest

from m3inputs import config_by_name, make_cotangents, make_scan_inputs, make_small_case
from oracle import grad
from tests._util import host, pooled_signed, rel_l2, tdev, to_device

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


def _run(m3, d, dy, dfin, io):
    dev = torch.device("cuda:0")
    iot = torch.float32 if io == "f32" else torch.bfloat16
    t = to_device(d, iot, torch.float32, dev)
    dyt = tdev(dy, iot, dev)
    dft = None if dfin is None else {k: tdev(v, torch.float32, dev) for k, v in dfin.items()}
    g = m3.scan_bwd(t["x"], t["B"], t["C"], t["dt"], t["lam"], t["theta"], t["A_log"], t["B_bias"], t["C_bias"],
                    t["init"], dyt, dfinal=dft, A_raw=t["A_raw"])
    torch.cuda.synchronize()
    return g


def _compare(g, want, d, tol, npairs):
    keys = [("x", "x"), ("B", "B"), ("C", "C"), ("dt", "dt"), ("lam", "lam")]
    if npairs:
        keys.append(("theta", "theta"))
    keys.append(("A", "A_raw" if d.get("A_raw") is not None else "A_log"))
    if d.get("B_bias") is not None:
        keys += [("B_bias", "B_bias"), ("C_bias", "C_bias")]
    errs = {}
    for gk, wk in keys:
        errs[gk] = rel_l2(host(g[gk]), want[wk])
    for k in ("h", "B_prev", "x_prev") + (("phi",) if npairs else ()):
        errs["init." + k] = rel_l2(host(g["init"][k]), want["init"][k])
    _say("  " + " ".join("%s %.1e" % kv for kv in errs.items()))
    for k, e in errs.items():
        assert e <= tol, (k, e)


CASES = [
    # name, small-case kwargs, io, final-carry sensitivities
    ("f32-P16N16-R2-G=H", dict(batch=2, seqlen=37, nheads=2, headdim=16, dstate=16, rank=2, npairs=4), "f32", True),
    ("f32-P8N12-R3-G1", dict(batch=1, seqlen=23, nheads=2, ngroups=1, headdim=8, dstate=12, rank=3, npairs=2),
     "f32", True),
    ("f32-heavy-R1-nocarry", dict(batch=2, seqlen=9, nheads=3, headdim=5, dstate=6, rank=1, npairs=0,
                                  init_full=False, bias=False, rate_dyn=True), "f32", False),
    ("f32-one-token", dict(batch=1, seqlen=1, nheads=2, headdim=4, dstate=8, rank=4, npairs=3), "f32", True),
    ("f32-R4-full-width", dict(batch=1, seqlen=19, nheads=2, ngroups=1, headdim=64, dstate=128, rank=4,
                               npairs=64), "f32", True),
    ("bf16-P64N128-R4-G1", dict(batch=2, seqlen=70, nheads=4, ngroups=1, headdim=64, dstate=128, rank=4,
                                npairs=32, rms_bc=True), "bf16", True),
    ("bf16-heavy-R2", dict(batch=1, seqlen=41, nheads=3, ngroups=1, headdim=64, dstate=128, rank=2, npairs=32,
                           rms_bc=True, rate_dyn=True), "bf16", False),
]


@pytest.mark.parametrize("name,kw,io,final", CASES, ids=[c[0] for c in CASES])
def test_scan_bwd_parity(m3, name, kw, io, final):
    _say("scan bwd", name)
    cfg, d = make_small_case(900 + len(name), io_dtype=io, **kw)
    dy, dfin = make_cotangents(cfg, seed=31, final=final)
    want = grad.scan_bwd(d, dy, dfin)
    g = _run(m3, d, dy, dfin, io)
    _compare(g, want, d, 1e-4 if io == "f32" else 2e-2, cfg.npairs)


# bf16 I/O at P 64, N 128, rank 4 runs the chunked matrix-core form (16-token chunks):
# ragged and single-token lengths, chunk edges, no rotation and all 64 pairs turning,
# heavy-tail rates, no carries, long memory over many chunks and steep decay.
CHUNKED = [
    ("one-token", dict(batch=1, seqlen=1, nheads=2, ngroups=1, npairs=32), True),
    ("one-chunk-all-pairs", dict(batch=2, seqlen=16, nheads=2, ngroups=2, npairs=64), True),
    ("chunk-plus-one", dict(batch=1, seqlen=17, nheads=3, ngroups=1, npairs=7), False),
    ("no-rotation-no-carry", dict(batch=2, seqlen=45, nheads=2, ngroups=1, npairs=0, init_full=False, bias=False), False),
    ("heavy-tail", dict(batch=1, seqlen=80, nheads=2, ngroups=1, npairs=32, rate_dyn=True), True),
    ("long-memory", dict(batch=1, seqlen=300, nheads=2, ngroups=1, npairs=16, dt_scale=1e-2), True),
    ("steep-decay", dict(batch=1, seqlen=64, nheads=2, ngroups=1, npairs=16, dt_scale=40.0), True),
]


@pytest.mark.parametrize("name,kw,final", CHUNKED, ids=[c[0] for c in CHUNKED])
def test_scan_bwd_chunked_form(m3, name, kw, final):
    _say("scan bwd chunked", name)
    cfg, d = make_small_case(1300 + len(name), io_dtype="bf16", headdim=64, dstate=128, rank=4, rms_bc=True, **kw)
    dy, dfin = make_cotangents(cfg, seed=41, final=final)
    want = grad.scan_bwd(d, dy, dfin)
    g = _run(m3, d, dy, dfin, "bf16")
    _compare(g, want, d, 2e-2, cfg.npairs)
    for gk, wk in (("x", "x"), ("B", "B"), ("dt", "dt")):
        assert abs(pooled_signed(host(g[gk]), want[wk])) <= 5e-3, gk


def test_scan_bwd_long_sequence(m3):
    """One batch of 64 heads in one group over 16,384 tokens (1,024 chunks per stream
    on the chunked form): the per-stream gradients (dx, dt, lambda, theta, the initial
    carry) of sampled streams against the oracle run on those streams alone.  The
    angle gradient is the one that would show rounding carried along the sequence."""
    cfg = config_by_name("mimo_bf16_prefill")
    d = make_scan_inputs(cfg, batch=1, seqlen=16384)
    dy, dfin = make_cotangents(cfg, seed=91, batch=1, seqlen=16384)
    _say("scan bwd long: inputs ready")
    g = _run(m3, d, dy, dfin, "bf16")
    for h in (0, 37):
        s = _one_stream(d, 0, h)
        sf = {k: v[0:1, h:h + 1] for k, v in dfin.items()}
        want = grad.scan_bwd(s, dy[0:1, :, h:h + 1], sf)
        errs = {"x": rel_l2(host(g["x"][0, :, h]), want["x"][0, :, 0]),
                "dt": rel_l2(host(g["dt"][0, :, h]), want["dt"][0, :, 0]),
                "lam": rel_l2(host(g["lam"][0, :, h]), want["lam"][0, :, 0]),
                "theta": rel_l2(host(g["theta"][0, :, h]), want["theta"][0, :, 0])}
        for k in ("h", "phi", "B_prev", "x_prev"):
            errs["init." + k] = rel_l2(host(g["init"][k][0, h]), want["init"][k][0, 0])
        _say("  stream (0, %d): " % h + " ".join("%s %.1e" % kv for kv in errs.items()))
        for k, e in errs.items():
            assert e <= 2e-2, (h, k, e)


def test_scan_bwd_empty_sequence(m3):
    """L = 0: the initial carry's gradients are the final carry's sensitivities."""
    cfg, d = make_small_case(5, batch=2, seqlen=0, nheads=2, headdim=4, dstate=8, rank=2, npairs=2)
    _, dfin = make_cotangents(cfg, seed=3)
    g = _run(m3, d, np.zeros((2, 0, 2, 2, 4), np.float32), dfin, "f32")
    for k in ("h", "phi", "B_prev", "x_prev"):
        assert np.array_equal(host(g["init"][k]), np.asarray(dfin[k], np.float64)), k
    assert np.all(host(g["A"]) == 0.0) and np.all(host(g["B_bias"]) == 0.0)


def _one_stream(d, bi, h):
    """The inputs of stream (bi, h) alone (G = 1: B and C are shared)."""
    s = {}
    for k in ("x", "dt", "lam", "theta", "A_raw"):
        v = d.get(k)
        s[k] = None if v is None else np.ascontiguousarray(v[bi:bi + 1, :, h:h + 1])
    s["B"] = d["B"][bi:bi + 1]
    s["C"] = d["C"][bi:bi + 1]
    s["A_log"] = d["A_log"][h:h + 1]
    for k in ("B_bias", "C_bias"):
        s[k] = None if d.get(k) is None else d[k][h:h + 1]
    s["init"] = None if d.get("init") is None else {k: v[bi:bi + 1, h:h + 1] for k, v in d["init"].items()}
    return s


def test_scan_bwd_prefill_full_size(m3):
    """The rank-4 prefill workload at full size (b 8, L 2048, H 64): the
    per-stream gradients (dx, dt, lambda, theta, initial carry) of sampled
    streams against the oracle run on those streams alone."""
    cfg = config_by_name("mimo_bf16_prefill")
    d = make_scan_inputs(cfg)
    dy, dfin = make_cotangents(cfg, seed=77)
    _say("scan bwd full size: inputs ready")
    g = _run(m3, d, dy, dfin, "bf16")
    for bi, h in [(0, 0), (5, 41), (7, 63)]:
        s = _one_stream(d, bi, h)
        sf = {k: v[bi:bi + 1, h:h + 1] for k, v in dfin.items()}
        want = grad.scan_bwd(s, dy[bi:bi + 1, :, h:h + 1], sf)
        errs = {"x": rel_l2(host(g["x"][bi, :, h]), want["x"][0, :, 0]),
                "dt": rel_l2(host(g["dt"][bi, :, h]), want["dt"][0, :, 0]),
                "lam": rel_l2(host(g["lam"][bi, :, h]), want["lam"][0, :, 0]),
                "theta": rel_l2(host(g["theta"][bi, :, h]), want["theta"][0, :, 0])}
        for k in ("h", "phi", "B_prev", "x_prev"):
            errs["init." + k] = rel_l2(host(g["init"][k][bi, h]), want["init"][k][0, 0])
        _say("  stream (%d, %d): " % (bi, h) + " ".join("%s %.1e" % kv for kv in errs.items()))
        for k, e in errs.items():
            assert e <= 2e-2, (bi, h, k, e)


def test_scan_bwd_all_heads_shared_gradients(m3):
    """One group shared by 64 heads (b 1, H 64, G 1, L 256, rank 4, bf16, rotation,
    bias, carries): the gradients summed across heads -- dB, dC (over the 64 heads
    of the group), d A_log (over tokens), the bias gradients -- and every per-head
    gradient, against the oracle over all heads.  The kernels sum dB and dC over
    heads with float atomics, so the order of the sums may change between runs:
    a second run must agree to float rounding (bounded), and so must a third."""
    cfg, d = make_small_case(31, batch=1, seqlen=256, nheads=64, ngroups=1, headdim=64, dstate=128, rank=4,
                             npairs=32, io_dtype="bf16", rms_bc=True, init_full=True)
    dy, dfin = make_cotangents(cfg, seed=3)
    want = grad.scan_bwd(d, dy, dfin)
    _say("  oracle done")
    g = _run(m3, d, dy, dfin, "bf16")
    _compare(g, want, d, 2e-2, cfg.npairs)
    for gk, wk in (("B", "B"), ("C", "C"), ("A", "A_log"), ("B_bias", "B_bias"), ("C_bias", "C_bias")):
        assert abs(pooled_signed(host(g[gk]), want[wk])) <= 5e-3, gk
    for _ in range(2):
        g2 = _run(m3, d, dy, dfin, "bf16")
        drift = {k: rel_l2(host(g2[k]), host(g[k])) for k in ("B", "C", "A", "B_bias", "C_bias", "x", "dt")}
        _say("  run-to-run drift: " + " ".join("%s %.1e" % kv for kv in drift.items()))
        for k, e in drift.items():
            assert e <= 2e-3, (k, e)


def test_scan_bwd_continuation(m3):
    """[DE] App C.2: gradients chain through the carries.  The backward of the
    second segment, with the whole sequence's final-carry sensitivities, gives the
    sensitivities of its initial carry; fed as the first segment's final-carry
    sensitivities, the two segments' gradients equal the whole sequence's (f32,
    rank 4, rotation, bias, 2 of 4 heads per group)."""
    cfg, d = make_small_case(77, batch=2, seqlen=150, nheads=4, ngroups=2, headdim=64, dstate=128, rank=4,
                             npairs=32, io_dtype="f32", rms_bc=True)
    dy, dfin = make_cotangents(cfg, seed=8)
    dev = torch.device("cuda:0")
    f32 = torch.float32
    t = to_device(d, f32, f32, dev)
    dyt = tdev(dy, f32, dev)
    dft = {k: tdev(v, f32, dev) for k, v in dfin.items()}
    whole = m3.scan_bwd(t["x"], t["B"], t["C"], t["dt"], t["lam"], t["theta"], t["A_log"], t["B_bias"], t["C_bias"],
                        t["init"], dyt, dfinal=dft)
    cut = 64
    sl = lambda v, a, b: None if v is None else v[:, a:b].contiguous()  # noqa: E731
    seg = [{k: sl(t[k], 0, cut) for k in ("x", "B", "C", "dt", "lam", "theta")},
           {k: sl(t[k], cut, 150) for k in ("x", "B", "C", "dt", "lam", "theta")}]
    _, mid = m3.scan_fwd(seg[0]["x"], seg[0]["B"], seg[0]["C"], seg[0]["dt"], seg[0]["lam"], seg[0]["theta"],
                         t["A_log"], t["B_bias"], t["C_bias"], t["init"], chunk=16, state_dtype=f32)
    g2 = m3.scan_bwd(seg[1]["x"], seg[1]["B"], seg[1]["C"], seg[1]["dt"], seg[1]["lam"], seg[1]["theta"], t["A_log"],
                     t["B_bias"], t["C_bias"], mid, dyt[:, cut:].contiguous(), dfinal=dft)
    g1 = m3.scan_bwd(seg[0]["x"], seg[0]["B"], seg[0]["C"], seg[0]["dt"], seg[0]["lam"], seg[0]["theta"], t["A_log"],
                     t["B_bias"], t["C_bias"], t["init"], dyt[:, :cut].contiguous(), dfinal=g2["init"])
    torch.cuda.synchronize()
    errs = {}
    for k in ("x", "B", "C", "dt", "lam", "theta"):
        errs[k] = rel_l2(np.concatenate([host(g1[k]), host(g2[k])], axis=1), host(whole[k]))
    for k in ("A", "B_bias", "C_bias"):
        errs[k] = rel_l2(host(g1[k]) + host(g2[k]), host(whole[k]))
    for k in ("h", "phi", "B_prev", "x_prev"):
        errs["init." + k] = rel_l2(host(g1["init"][k]), host(whole["init"][k]))
    _say("  continuation: " + " ".join("%s %.1e" % kv for kv in errs.items()))
    for k, e in errs.items():
        assert e <= 1e-4, (k, e)


def test_scan_bwd_bf16_state_and_groups(m3):
    """A bf16 initial state (the decode workload's state dtype) and two groups of
    two heads, against the oracle."""
    cfg, d = make_small_case(404, batch=2, seqlen=33, nheads=4, ngroups=2, headdim=64, dstate=128, rank=2,
                             npairs=16, io_dtype="bf16", state_dtype="bf16", rms_bc=True)
    dy, dfin = make_cotangents(cfg, seed=9)
    want = grad.scan_bwd(d, dy, dfin)
    dev = torch.device("cuda:0")
    t = to_device(d, torch.bfloat16, torch.bfloat16, dev)
    g = m3.scan_bwd(t["x"], t["B"], t["C"], t["dt"], t["lam"], t["theta"], t["A_log"], t["B_bias"], t["C_bias"],
                    t["init"], tdev(dy, torch.bfloat16, dev),
                    dfinal={k: tdev(v, torch.float32, dev) for k, v in dfin.items()}, state_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    _compare(g, want, d, 2e-2, cfg.npairs)


def _sweep_cases(n=12, seed=2027):
    """Seeded random small shapes over what the backward supports (P <= 64, N <= 128,
    R <= 4, any npairs <= N/2, groups dividing the heads, both rate laws, carries or
    not, ragged lengths, both I/O dtypes)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        P = int(rng.choice([3, 8, 16, 33, 64]))
        N = int(rng.choice([2, 6, 16, 40, 128]))
        R = int(rng.integers(1, 5))
        H = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([g for g in (1, 2, 4) if H % g == 0]))
        c = dict(P=P, N=N, R=R, H=H, G=G, npairs=int(rng.integers(0, N // 2 + 1)),
                 L=int(rng.integers(1, 41)), io=str(rng.choice(["f32", "bf16"])),
                 heavy=bool(rng.integers(0, 2)), init=bool(rng.integers(0, 2)), final=bool(rng.integers(0, 2)))
        if c["L"] == 1:
            # one token and no carry: the angle gradient is zero by rotation invariance
            # (test_scan_bwd_angle_invariance); keep a carry so that it is not
            c["init"] = True
        out.append(c)
    return out


@pytest.mark.parametrize("c", _sweep_cases(), ids=lambda c: "P%(P)d-N%(N)d-R%(R)d-H%(H)d-G%(G)d-np%(npairs)d-L%(L)d-%(io)s" % c)
def test_scan_bwd_random_shapes(m3, c):
    """Every gradient against the oracle on a seeded random shape, plus the
    pooled signed error sum(gpu - oracle) / ||oracle||_1 as a bias check ([DE]
    App C.4), at a quarter of the normwise tolerance."""
    cfg, d = make_small_case(7000 + c["P"] + 3 * c["N"] + c["L"], batch=2, seqlen=c["L"], nheads=c["H"],
                             ngroups=c["G"], headdim=c["P"], dstate=c["N"], rank=c["R"], npairs=c["npairs"],
                             io_dtype=c["io"], init_full=c["init"], rate_dyn=c["heavy"])
    dy, dfin = make_cotangents(cfg, seed=12, final=c["final"])
    want = grad.scan_bwd(d, dy, dfin)
    g = _run(m3, d, dy, dfin, c["io"])
    tol = 1e-4 if c["io"] == "f32" else 2e-2
    _compare(g, want, d, tol, cfg.npairs)
    for gk, wk in (("x", "x"), ("B", "B"), ("dt", "dt")):
        assert abs(pooled_signed(host(g[gk]), want[wk])) <= tol / 4, gk


def test_scan_bwd_angle_invariance(m3):
    """One token and no carry: B and C turn by the same angle, so every C . B product
    and the output do not depend on it, and the angle gradients vanish (to rounding)."""
    cfg, d = make_small_case(11, batch=2, seqlen=1, nheads=2, headdim=33, dstate=128, rank=2, npairs=45,
                             io_dtype="f32", init_full=False)
    dy, _ = make_cotangents(cfg, seed=4, final=False)
    g = _run(m3, d, dy, None, "f32")
    scale = float(np.abs(host(g["B"])).max())
    assert float(np.abs(host(g["theta"])).max()) <= 1e-5 * scale
    assert float(np.abs(host(g["init"]["phi"])).max()) <= 1e-5 * scale
