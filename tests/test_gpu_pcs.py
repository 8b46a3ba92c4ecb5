"""GPU parity of the per-coordinate selective scan (m3_pcs_fwd, the Mamba 1
preset) against the fp64 C oracle (``oracle.pcs_cpu``), element by element.

Bound.  The kernel keeps the state and every sum in fp32 and rounds y once to
the I/O dtype (round to nearest even).  Per element,
    |y_gpu - y_oracle| <= rel |y_oracle| + abs_frac rms(y_oracle)
with rel = 2^-8 + 3e-5 for bf16 output (half a bf16 ulp is up to 2^-8 of the
value, at the bottom of a binade; 3e-5 for the fp32 arithmetic before the
rounding) and 3e-5 for fp32 output; the absolute part covers the fp32 sums near a zero of y
(cancellation among the N products C h): abs_frac = 1e-4 (bf16), 3e-5 (fp32).
The final state is fp32 on both sides: |h_gpu - h_oracle| <= 3e-5 (|h| +
rms(h)).  A dropped term, a wrong coordinate, token or group scores O(1).

Long memory.  Each step's decay exp(dt a) carries a relative error of about
2.5e-7 in fp32 (the exponent's product, the exp2 instruction's ulp, the fma),
and a state that remembers M tokens compounds M of them: every relative bound
above grows by 2.5e-7 M, with M = min(L, 1 / (mean(dt) min|a|)) the longest
memory of the case (about 8 tokens under the default step law, thousands in the
long-memory cases).
"""
import sys

import numpy as np
import pytest

from m3inputs.pcs import PCS_CONFIGS, make_pcs_inputs
from oracle import pcs_cpu

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


def _dev(inp, io, dev):
    t = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev).to(dt)  # noqa: E731
    return dict(x=t(inp["x"], io), dt=t(inp["dt"], torch.float32), A_log=t(inp["A_log"], torch.float32),
                B=t(inp["B"], io), C=t(inp["C"], io), h0=t(inp["h0"], torch.float32))


def _bound_excess(g, r, rel, abs_frac):
    """max over elements of |g - r| / (rel |r| + abs_frac rms(r)); <= 1 passes."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r))) or 1.0
    return float((np.abs(g - r) / (rel * np.abs(r) + abs_frac * rms)).max())


def _memory(inp):
    """The case's longest state memory in tokens (for the fp32 drift term)."""
    L = inp["x"].shape[1]
    amin = float(np.exp(np.asarray(inp["A_log"], np.float64)).min())
    mdt = float(np.mean(inp["dt"])) if inp["dt"].size else 1.0
    return min(float(L), 1.0 / (mdt * amin))


def _tols(io, inp):
    """(rel_y, abs_y, rel_h)"""
    drift = 2.5e-7 * _memory(inp)
    if io == torch.bfloat16:
        return 2.0 ** -8 + 3e-5 + drift, 1e-4 + drift, 3e-5 + drift
    return 3e-5 + drift, 3e-5 + drift, 3e-5 + drift


def _run_and_compare(m3, inp, io, nsegments=0, label=""):
    dev = torch.device("cuda:0")
    t = _dev(inp, io, dev)
    _say("pcs case", label, "x", tuple(inp["x"].shape), "N", inp["A_log"].shape[1], "G", inp["B"].shape[2],
         "io", io, "nseg", nsegments, "h0", inp["h0"] is not None)
    y, h1 = m3.pcs_fwd(t["x"], t["dt"], t["A_log"], t["B"], t["C"], t["h0"], nsegments=nsegments)
    torch.cuda.synchronize()
    yr, hr = pcs_cpu.scan(inp, inp["h0"])
    rel, af, rh = _tols(io, inp)
    ey = _bound_excess(y.float().cpu().numpy(), yr, rel, af)
    eh = _bound_excess(h1.cpu().numpy(), hr, rh, rh)
    _say("   y excess %.3f  h excess %.3f" % (ey, eh))
    assert ey <= 1.0, (label, ey)
    assert eh <= 1.0, (label, eh)


SMALL = [
    # (batch, L, D, G, N, io, init, nseg)
    (2, 200, 200, 1, 16, "bf16", False, 0),      # ragged tokens (6 blocks + 8) and channels (3 tiles + 8)
    (1, 64, 64, 1, 8, "bf16", True, 0),          # one block, one tile
    (2, 130, 256, 2, 32, "bf16", True, 0),       # two groups of 128 channels
    (1, 77, 128, 1, 64, "bf16", True, 0),
    (2, 150, 100, 1, 16, "f32", True, 0),        # f32 I/O, ragged channels (100 = 64 + 36)
    (1, 65, 256, 4, 8, "f32", False, 0),         # four groups of 64 channels
    (1, 1, 64, 1, 16, "bf16", True, 0),          # a single token
    (2, 1000, 128, 1, 16, "bf16", True, 5),      # segmented: 5 segments of 224 tokens (last one ragged)
    (1, 640, 64, 1, 32, "f32", True, 64),        # 64 requested, clamped to 20 one-block segments
    (1, 3000, 64, 1, 64, "bf16", True, 64),      # 64 requested: 47 segments of 64 tokens
    (1, 96, 128, 2, 8, "bf16", True, 3),         # three one-block segments, two groups
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "b%d_L%d_D%d_G%d_N%d_%s_h0%d_s%d" % c)
def test_pcs_small(m3, case):
    b, L, D, G, N, io, init, nseg = case
    inp = make_pcs_inputs(batch=b, channels=D, seqlen=L, dstate=N, ngroups=G, io=io, seed=7000 + L + D + N,
                          init=init)
    _run_and_compare(m3, inp, torch.bfloat16 if io == "bf16" else torch.float32, nseg, "small")


@pytest.mark.parametrize("nseg", [1, 7, 64])
def test_pcs_long_memory_segments(m3, nseg):
    """Steps 1000 times smaller (per-step decay exp(-1.3e-4 .. -2e-3)): the state
    remembers thousands of tokens, so each segment's incoming state (the carry
    pass's prefix scan over segments) decides the outputs."""
    inp = make_pcs_inputs(batch=2, channels=128, seqlen=6000, dstate=16, io="bf16", seed=7101, init=True,
                          dt_scale=1e-3)
    _run_and_compare(m3, inp, torch.bfloat16, nseg, "long-memory")


def test_pcs_empty_sequence(m3):
    """L = 0: the final state is the initial one (zeros without one); y is empty."""
    dev = torch.device("cuda:0")
    inp = make_pcs_inputs(batch=2, channels=64, seqlen=0, dstate=16, io="bf16", seed=7201, init=True)
    t = _dev(inp, torch.bfloat16, dev)
    y, h1 = m3.pcs_fwd(t["x"], t["dt"], t["A_log"], t["B"], t["C"], t["h0"])
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.equal(h1, t["h0"])
    _, h2 = m3.pcs_fwd(t["x"], t["dt"], t["A_log"], t["B"], t["C"], None)
    torch.cuda.synchronize()
    assert torch.count_nonzero(h2).item() == 0


def test_pcs_schedule_independence(m3):
    """The segment count changes rounding only: 1, 3 and 16 segments agree with
    each other to fp32 noise on bf16-exact inputs, f32 output."""
    dev = torch.device("cuda:0")
    inp = make_pcs_inputs(batch=1, channels=64, seqlen=2048, dstate=16, io="f32", seed=7301, init=True,
                          dt_scale=1e-2)
    t = _dev(inp, torch.float32, dev)
    ys = [m3.pcs_fwd(t["x"], t["dt"], t["A_log"], t["B"], t["C"], t["h0"], nsegments=k)[0] for k in (1, 3, 16)]
    torch.cuda.synchronize()
    rel, af, _ = _tols(torch.float32, inp)
    for yk in ys[1:]:
        assert _bound_excess(yk.cpu().numpy(), ys[0].cpu().numpy(), 2 * rel, 2 * af) <= 1.0


@pytest.mark.parametrize("name", sorted(PCS_CONFIGS))
def test_pcs_full_size(m3, name):
    """The timing workloads at their full sizes, in the schedule the benchmark
    runs (the library's segment choice): every channel of every batch against
    the oracle, in slabs of channels."""
    cfg = dict(PCS_CONFIGS[name])
    io = torch.bfloat16 if cfg.pop("io") == "bf16" else torch.float32
    seed = cfg.pop("seed")
    inp = make_pcs_inputs(**cfg, io="bf16" if io == torch.bfloat16 else "f32", seed=seed, init=True)
    dev = torch.device("cuda:0")
    t = _dev(inp, io, dev)
    _say("pcs full", name, cfg)
    y, h1 = m3.pcs_fwd(t["x"], t["dt"], t["A_log"], t["B"], t["C"], t["h0"])
    torch.cuda.synchronize()
    yg = y.float().cpu().numpy()
    hg = h1.cpu().numpy()
    del t, y, h1
    D = cfg["channels"]
    rel, af, rh = _tols(io, inp)
    slab = 512
    worst_y = worst_h = 0.0
    # the rms scale of the absolute term is that of the whole output
    rms_parts = []
    refs = []
    for d0 in range(0, D, slab):
        yr, hr = pcs_cpu.scan(inp, inp["h0"], d0, min(D, d0 + slab))
        rms_parts.append(float(np.mean(yr * yr)))
        refs.append((d0, yr.astype(np.float32), hr))
    rms_y = float(np.sqrt(np.mean(rms_parts)))
    for d0, yr, hr in refs:
        d1 = d0 + yr.shape[2]
        g = yg[:, :, d0:d1].astype(np.float64)
        r = yr.astype(np.float64)
        worst_y = max(worst_y, float((np.abs(g - r) / (rel * np.abs(r) + af * rms_y)).max()))
        worst_h = max(worst_h, _bound_excess(hg[:, d0:d1], hr, rh, rh))
    _say("   %s: y excess %.3f  h excess %.3f" % (name, worst_y, worst_h))
    assert worst_y <= 1.0
    assert worst_h <= 1.0
