"""The no-allocation scan entry point (m3_scan_fwd_noalloc, through the C ABI)
against m3_scan_fwd on the same inputs: calls in a row, each with a smaller input
than the one before, on shapes whose schedule uses the workspace (the segmented
schedule's summaries; the single-rank path's score tiles).  The
two entry points run the same kernels and schedule, so their results agree bit
for bit; both also meet the workload tolerance against the fp64 oracle."""
import sys

import numpy as np
import pytest

from m3inputs import make_small_case
from oracle import ref_cpu
from tests._util import host, phase_err, rel_l2, to_device

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def m3():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_mimo_amd as m
    return m


CASES = [  # (seed, small-case kwargs): the larger first, then a smaller one with another rank and chunk
    (71, dict(batch=1, seqlen=1000, nheads=4, ngroups=1, headdim=64, dstate=128, rank=4, npairs=32, chunk=64)),
    (72, dict(batch=1, seqlen=300, nheads=2, ngroups=1, headdim=64, dstate=128, rank=2, npairs=16, chunk=32)),
    # the single-rank path (no rotation, no bias): its workspace holds the head-shared score tiles
    (73, dict(batch=1, seqlen=200, nheads=2, ngroups=1, headdim=64, dstate=128, rank=1, npairs=0, chunk=64,
              bias=False)),
]


def test_noalloc_matches_scan_fwd(m3):
    dev = torch.device("cuda:0")
    bf, f32 = torch.bfloat16, torch.float32
    for seed, kw in CASES:
        print("case", seed, kw, flush=True)
        cfg, d = make_small_case(seed, io_dtype="bf16", rms_bc=True, init_full=True, **kw)
        t = to_device(d, bf, f32, dev)
        desc = m3.make_desc(t["x"], t["B"], t["theta"], chunk=cfg.chunk, state_dtype=f32)
        need = m3.scan_workspace_size(desc)
        assert 0 < need <= m3.lib.m3_scan_noalloc_max_workspace(), need     # the scratch is in use
        b, L, H, R, P = t["x"].shape
        args = (t["x"], t["B"], t["C"], t["dt"], t["lam"], t["theta"], t["A_log"], t["B_bias"], t["C_bias"], t["init"])
        y_ref, f_ref = m3.scan_fwd(*args, chunk=cfg.chunk)
        y = torch.full_like(t["x"], float("nan"))
        fin = m3.new_carry(b, H, P, cfg.dstate, R, cfg.npairs, bf, f32, dev)
        m3.scan_fwd_noalloc(*args, y=y, final=fin, chunk=cfg.chunk)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
        for k in ("h", "phi", "B_prev", "x_prev"):
            assert torch.equal(fin[k], f_ref[k]), k
        yr, fr = ref_cpu.scan(d)
        e = rel_l2(host(y), yr)
        eh = rel_l2(host(fin["h"]), fr["h"])
        print("  noalloc: y rel-L2 %.2e, h rel-L2 %.2e (workspace %d bytes)" % (e, eh, need), flush=True)
        assert e <= 2e-2 and eh <= 2e-2
        assert rel_l2(host(fin["B_prev"]), fr["B_prev"]) <= 2e-2
        assert phase_err(host(fin["phi"]), fr["phi"]) < 1e-3
    sys.stdout.flush()
