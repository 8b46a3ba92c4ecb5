"""GPU parity on the five workloads at their full sizes.

The oracle (fp64 C recurrence) runs on a sample of whole (batch, head)
streams -- streams are independent, so every sampled output is exact -- and
the GPU result of those streams is compared element by element.
"""
import sys
import time

import numpy as np
import pytest

from m3inputs import config_by_name, make_scan_inputs
from oracle import ref_cpu
from tests._util import host, phase_err, pooled_signed, rel_l2

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


def _scan_full(m3, cfg, sel, nsegments=0):
    t0 = time.time()
    d = make_scan_inputs(cfg)
    _say("  %s: inputs %.1fs" % (cfg.name, time.time() - t0))
    dev = torch.device("cuda:0")
    io = torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32

    def T(a, dt):
        return None if a is None else torch.from_numpy(a).to(dev).to(dt)
    init = None
    if d["init"] is not None:
        init = {"h": T(d["init"]["h"], torch.float32), "phi": T(d["init"]["phi"], torch.float32),
                "B_prev": T(d["init"]["B_prev"], io), "x_prev": T(d["init"]["x_prev"], io)}
    y, fin = m3.scan_fwd(T(d["x"], io), T(d["B"], io), T(d["C"], io), T(d["dt"], torch.float32),
                         T(d["lam"], torch.float32), T(d["theta"], torch.float32), T(d["A_log"], torch.float32),
                         T(d["B_bias"], torch.float32), T(d["C_bias"], torch.float32), init, chunk=cfg.chunk,
                         nsegments=nsegments)
    torch.cuda.synchronize()
    _say("  %s: gpu done %.1fs" % (cfg.name, time.time() - t0))
    yr, fr = ref_cpu.scan(d, sel=sel)
    _say("  %s: oracle on %d streams %.1fs" % (cfg.name, len(sel), time.time() - t0))
    tol = 1e-4 if cfg.io_dtype == "f32" else 2e-2
    for i, (bi, h) in enumerate(sel):
        yg = host(y[bi, :, h])
        e = rel_l2(yg, yr[i])
        eh = rel_l2(host(fin["h"][bi, h]), fr["h"][i])
        ps = pooled_signed(yg, yr[i])
        _say("  stream (%d,%d): y rel-L2 %.3e (signed %.1e), h rel-L2 %.3e" % (bi, h, e, ps, eh))
        assert e <= tol and eh <= tol and abs(ps) <= tol / 4
        assert rel_l2(host(fin["B_prev"][bi, h]), fr["B_prev"][i]) <= tol
        assert rel_l2(host(fin["x_prev"][bi, h]), fr["x_prev"][i]) <= tol
        if cfg.npairs:
            assert phase_err(host(fin["phi"][bi, h]), fr["phi"][i]) < 1e-3
    assert torch.isfinite(y.float()).all()


def test_config2_siso_bf16(m3):
    _scan_full(m3, config_by_name("siso_bf16_mamba2"), [(0, 0), (1, 17), (3, 31), (2, 5)])


def test_config3_mimo_prefill(m3):
    _scan_full(m3, config_by_name("mimo_bf16_prefill"), [(0, 0), (7, 63), (3, 40), (5, 11)])


def test_config5_long_context(m3):
    _scan_full(m3, config_by_name("mimo_bf16_long"), [(0, 0), (0, 37), (0, 63)])


def test_config4_decode_1000_steps(m3):
    """1000 consecutive in-place decode steps at batch 256, 64 heads; the
    oracle replays sampled streams over the same 1000 steps."""
    from m3inputs.gen_torch import decode_inputs_device, stream_inputs_host
    cfg = config_by_name("mimo_bf16_decode")
    dev = torch.device("cuda:0")
    S = cfg.decode_steps
    d = decode_inputs_device(cfg, S, dev, cfg.seed)
    b, H, R, P, N = cfg.batch, cfg.nheads, cfg.rank, cfg.headdim, cfg.dstate
    carry = m3.new_carry(b, H, P, N, R, cfg.npairs, torch.bfloat16, torch.bfloat16, dev)
    carry["h"].copy_(d["h0"])
    sel = [(0, 0), (255, 63), (100, 7), (31, 32)]
    ysel = torch.empty((S, len(sel), R, P), dtype=torch.bfloat16, device=dev)
    y = torch.empty((b, H, R, P), dtype=torch.bfloat16, device=dev)
    for s in range(S):
        m3.decode_step(d["x"][s], d["B"][s], d["C"][s], d["dt"][s], d["lam"][s], d["theta"][s], d["A_log"],
                       d["B_bias"], d["C_bias"], carry, y=y)
        for i, (bi, h) in enumerate(sel):
            ysel[s, i] = y[bi, h]
    torch.cuda.synchronize()
    _say("  decode: 1000 steps done")
    for i, (bi, h) in enumerate(sel):
        hin = stream_inputs_host(d, bi, h, G=cfg.ngroups, H=H)
        yr, fr = ref_cpu.scan(hin)
        e = rel_l2(host(ysel[:, i]), yr[0, :, 0])
        eh = rel_l2(host(carry["h"][bi, h]), fr["h"][0, 0])
        _say("  stream (%d,%d): y rel-L2 %.3e, h rel-L2 %.3e" % (bi, h, e, eh))
        assert e <= 2e-2 and eh <= 2e-2
        assert rel_l2(host(carry["B_prev"][bi, h]), fr["B_prev"][0, 0]) <= 2e-2
        assert phase_err(host(carry["phi"][bi, h]), fr["phi"][0, 0]) < 1e-3
