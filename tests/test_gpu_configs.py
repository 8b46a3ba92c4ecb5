"""GPU parity on the five workloads at their full sizes.

The scan workloads are compared on EVERY (batch, head) stream: the oracle (fp64
C recurrence) runs all streams in batches, and each stream's outputs and final
carry are compared element by element.  Three bounds apply to each stream:
  * the normwise relative L2 error of its whole output tensor (2e-2 for bf16
    I/O, the workload tolerance), and the same for each final-carry member;
  * the pooled signed error sum(gpu - oracle) / ||oracle||_1 (a bias check);
  * a per-row bound: every (token, rank) row of P outputs separately, with the
    error norm divided by max(||row||, half the stream's RMS row norm).
    One wrong row would add only about sqrt(1 / (L R)) to the whole-tensor
    error, which the first bound cannot see; here it scores about 1.
The decode workload replays one stream of every head (64 streams spread over
the batch) through the same 1000 steps on the oracle.
"""
import sys
import time

import numpy as np
import pytest

from m3inputs import config_by_name, make_scan_inputs
from oracle import ref_cpu
from tests._util import ROW_TOL, host, phase_err, pooled_signed, rel_l2, row_errors

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


def compare_streams(cfg, d, y_host, fin_host, nbatch):
    """Every stream of a scan workload against the oracle, nbatch streams at a time."""
    b, H = cfg.batch, cfg.nheads
    tol = 1e-4 if cfg.io_dtype == "f32" else 2e-2
    sel_all = [(bi, h) for bi in range(b) for h in range(H)]
    worst = {"y": 0.0, "row": 0.0, "row_f0.1": 0.0, "row_f1": 0.0, "signed": 0.0, "h": 0.0, "B_prev": 0.0,
             "x_prev": 0.0, "phi": 0.0}
    where = {}
    t0 = time.time()
    for s0 in range(0, len(sel_all), nbatch):
        sel = sel_all[s0:s0 + nbatch]
        yr, fr = ref_cpu.scan(d, sel=sel)
        for i, (bi, h) in enumerate(sel):
            yg = y_host[bi, :, h]
            e = {"y": rel_l2(yg, yr[i]), "signed": abs(pooled_signed(yg, yr[i])),
                 "row": float(row_errors(yg, yr[i]).max()) if yg.size else 0.0,
                 "row_f0.1": float(row_errors(yg, yr[i], 0.1).max()) if yg.size else 0.0,
                 "row_f1": float(row_errors(yg, yr[i], 1.0).max()) if yg.size else 0.0,
                 "h": rel_l2(fin_host["h"][bi, h], fr["h"][i]),
                 "B_prev": rel_l2(fin_host["B_prev"][bi, h], fr["B_prev"][i]),
                 "x_prev": rel_l2(fin_host["x_prev"][bi, h], fr["x_prev"][i]),
                 "phi": phase_err(fin_host["phi"][bi, h], fr["phi"][i]) if cfg.npairs else 0.0}
            for k, v in e.items():
                if v > worst[k]:
                    worst[k], where[k] = v, (bi, h)
            assert e["y"] <= tol and e["h"] <= tol and e["B_prev"] <= tol and e["x_prev"] <= tol, ((bi, h), e)
            assert e["signed"] <= tol / 4, ((bi, h), e)
            assert e["row"] <= (ROW_TOL if cfg.io_dtype == "bf16" else 1e-3), ((bi, h), e)
            assert e["phi"] < 1e-3, ((bi, h), e)
        _say("  %s: %d/%d streams compared (%.1fs)" % (cfg.name, s0 + len(sel), len(sel_all), time.time() - t0))
    _say("  %s worst over all %d streams: " % (cfg.name, len(sel_all)) +
         " ".join("%s %.2e at %s" % (k, worst[k], where.get(k)) for k in worst))
    return worst


def _scan_full(m3, cfg, nbatch, nsegments=0):
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
    assert torch.isfinite(y.float()).all()
    y_host = y.float().cpu().numpy()
    fin_host = {k: v.float().cpu().numpy() for k, v in fin.items()}
    del y, fin
    torch.cuda.empty_cache()
    _say("  %s: gpu done %.1fs" % (cfg.name, time.time() - t0))
    return compare_streams(cfg, d, y_host, fin_host, nbatch)


def test_config2_siso_bf16(m3):
    _scan_full(m3, config_by_name("siso_bf16_mamba2"), nbatch=128)


def test_config3_mimo_prefill(m3):
    _scan_full(m3, config_by_name("mimo_bf16_prefill"), nbatch=128)


def test_config5_long_context(m3):
    _scan_full(m3, config_by_name("mimo_bf16_long"), nbatch=16)


def test_config4_decode_1000_steps(m3):
    """1000 consecutive in-place decode steps at batch 256, 64 heads; the
    oracle replays one stream of every head (spread over the batch) over the
    same 1000 steps."""
    from m3inputs.gen_torch import decode_inputs_device, stream_inputs_host
    cfg = config_by_name("mimo_bf16_decode")
    dev = torch.device("cuda:0")
    S = cfg.decode_steps
    d = decode_inputs_device(cfg, S, dev, cfg.seed)
    b, H, R, P, N = cfg.batch, cfg.nheads, cfg.rank, cfg.headdim, cfg.dstate
    carry = m3.new_carry(b, H, P, N, R, cfg.npairs, torch.bfloat16, torch.bfloat16, dev)
    carry["h"].copy_(d["h0"])
    sel = [((97 * h + 13) % b, h) for h in range(H)] + [(0, 0), (255, 63), (100, 7), (31, 32)]
    bsel = torch.tensor([s[0] for s in sel], device=dev)
    hsel = torch.tensor([s[1] for s in sel], device=dev)
    ysel = torch.empty((S, len(sel), R, P), dtype=torch.bfloat16, device=dev)
    y = torch.empty((b, H, R, P), dtype=torch.bfloat16, device=dev)
    for s in range(S):
        m3.decode_step(d["x"][s], d["B"][s], d["C"][s], d["dt"][s], d["lam"][s], d["theta"][s], d["A_log"],
                       d["B_bias"], d["C_bias"], carry, y=y)
        ysel[s] = y[bsel, hsel]
    torch.cuda.synchronize()
    _say("  decode: 1000 steps done")
    worst_y = worst_row = 0.0
    for i, (bi, h) in enumerate(sel):
        hin = stream_inputs_host(d, bi, h, G=cfg.ngroups, H=H)
        yr, fr = ref_cpu.scan(hin)
        yg = host(ysel[:, i])
        e = rel_l2(yg, yr[0, :, 0])
        er = float(row_errors(yg, yr[0, :, 0]).max())
        eh = rel_l2(host(carry["h"][bi, h]), fr["h"][0, 0])
        worst_y, worst_row = max(worst_y, e), max(worst_row, er)
        assert e <= 2e-2 and eh <= 2e-2 and er <= ROW_TOL, ((bi, h), e, eh, er)
        assert rel_l2(host(carry["B_prev"][bi, h]), fr["B_prev"][0, 0]) <= 2e-2
        assert rel_l2(host(carry["x_prev"][bi, h]), fr["x_prev"][0, 0]) <= 2e-2
        assert phase_err(host(carry["phi"][bi, h]), fr["phi"][0, 0]) < 1e-3
    _say("  decode: %d streams (every head), worst y rel-L2 %.2e, worst row %.2e" % (len(sel), worst_y, worst_row))
