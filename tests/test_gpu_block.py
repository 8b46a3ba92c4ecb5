"""GPU parity of the layer entry points (m3_block_fwd, m3_block_decode_step,
through the C ABI) against the fp64 layer oracle (``oracle.block``).

Tolerances (normwise relative L2 per tensor): 1e-4 for f32 I/O, 2e-2 for bf16.
"""
import sys

import numpy as np
import pytest

from m3inputs import config_by_name, make_block_inputs
from oracle import block
from tests._util import ROW_TOL, host, phase_err, rel_l2, row_errors, tdev

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


def _dev_block(d, io):
    dev = torch.device("cuda:0")
    t = {k: tdev(d[k], io, dev) for k in ("z", "x", "B_raw", "C_raw")}
    for k in ("dt_raw", "A_raw", "lam_raw", "th_raw"):
        t[k] = tdev(d.get(k), torch.float32, dev)
    t["params"] = {k: tdev(v, torch.float32, dev) for k, v in d["params"].items()}
    t["params"]["eps"] = block.RMS_EPS
    if d.get("init") is not None:
        i = d["init"]
        t["init"] = {"h": tdev(i["h"], torch.float32, dev), "phi": tdev(i["phi"], torch.float32, dev),
                     "B_prev": tdev(i["B_prev"], io, dev), "x_prev": tdev(i["x_prev"], io, dev)}
    else:
        t["init"] = None
    return t


CASES = [
    # io,   P,  N,   R, np, G, Q,  L
    ("f32", 16, 16, 2, 4, 1, 16, 37),
    ("f32", 8, 12, 3, 0, 2, 5, 23),
    ("bf16", 64, 128, 4, 32, 1, 64, 150),
    ("bf16", 64, 128, 4, 32, 1, 16, 90),
    ("bf16", 64, 128, 1, 0, 1, 64, 130),
    # the other fused layouts: each consumer's output pieces in one or two lane slots
    ("bf16", 64, 128, 2, 32, 1, 32, 100),
    ("bf16", 64, 128, 2, 16, 1, 64, 140),
    ("bf16", 64, 128, 4, 32, 1, 32, 70),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-P%d-N%d-R%d-np%d-G%d-Q%d-L%d" % c)
def test_block_fwd(m3, case):
    io, P, N, R, npairs, G, Q, L = case
    _say("block fwd", case)
    cfg = config_by_name("tiny_siso_f32").with_(batch=2, seqlen=L, nheads=4, ngroups=G, headdim=P, dstate=N,
                                                rank=R, npairs=npairs, chunk=Q, io_dtype=io, state_dtype="f32")
    d = make_block_inputs(cfg, seed=6000 + P + R + Q + L)
    want, wfin = block.block_forward(d)
    iot = torch.float32 if io == "f32" else torch.bfloat16
    t = _dev_block(d, iot)
    out, fin = m3.block_fwd(t["z"], t["x"], t["B_raw"], t["C_raw"], t["dt_raw"], t["A_raw"], t["lam_raw"],
                            t["th_raw"], t["params"], t["init"], chunk=Q)
    torch.cuda.synchronize()
    tol = 1e-4 if io == "f32" else 2e-2
    e = rel_l2(host(out), want)
    # every (token, head) row of P outputs on its own, so that one wrong row or piece
    # cannot hide under the tensor norm
    er = float(row_errors(host(out), want).max()) if want.size else 0.0
    _say("  out rel-L2 %.3e  worst row %.3e" % (e, er))
    assert e <= tol
    assert er <= (5e-4 if io == "f32" else ROW_TOL)
    for k in ("h", "B_prev", "x_prev"):
        ek = rel_l2(host(fin[k]), wfin[k])
        _say("  %s rel-L2 %.3e" % (k, ek))
        assert ek <= tol, k
    if npairs:
        assert phase_err(host(fin["phi"]), wfin["phi"]) < 1e-3


@pytest.mark.parametrize("io,P,N,R,npairs,steps", [("f32", 16, 16, 2, 4, 5), ("bf16", 64, 128, 4, 32, 6)])
def test_block_decode_steps(m3, io, P, N, R, npairs, steps):
    """k layer decode steps equal the layer oracle over k tokens (output and
    carried state, phase, previous write)."""
    _say("block decode", io, P, N, R, npairs, steps)
    cfg = config_by_name("tiny_siso_f32").with_(batch=3, seqlen=steps, nheads=4, ngroups=1, headdim=P, dstate=N,
                                                rank=R, npairs=npairs, io_dtype=io, state_dtype="f32")
    d = make_block_inputs(cfg, seed=6100 + P)
    want, wfin = block.block_forward(d)
    iot = torch.float32 if io == "f32" else torch.bfloat16
    t = _dev_block(d, iot)
    carry = {k: v.clone() for k, v in t["init"].items()}
    outs = []
    for s in range(steps):
        tok = {k: (None if t[k] is None else t[k][:, s].contiguous())
               for k in ("z", "x", "B_raw", "C_raw", "dt_raw", "A_raw", "lam_raw", "th_raw")}
        outs.append(m3.block_decode_step(tok["z"], tok["x"], tok["B_raw"], tok["C_raw"], tok["dt_raw"], tok["A_raw"],
                                         tok["lam_raw"], tok["th_raw"], t["params"], carry))
    torch.cuda.synchronize()
    tol = 1e-4 if io == "f32" else 2e-2
    e = rel_l2(host(torch.stack(outs, dim=1)), want)
    _say("  out rel-L2 %.3e" % e)
    assert e <= tol
    for k in ("h", "B_prev", "x_prev"):
        assert rel_l2(host(carry[k]), wfin[k]) <= tol, k
