"""Seeded inputs of the per-coordinate selective scan (the Mamba 1 preset).

Value laws: x ~ N(0, 1); dt = softplus(N(-2, 0.5)) per (b, t, channel);
A_log = log U(1, 16) per (channel, coordinate) (the scan's static rates are
-exp(A_log)); B, C ~ N(0, 1) per (b, t, group, coordinate); h0 ~ N(0, 0.1).
x, B, C are rounded to the I/O dtype (bf16 by round-to-nearest-even) so that
the oracle and the GPU see identical values.  Input preparation only: none of
the recurrence's arithmetic is here.
"""
import numpy as np

from .gen import bf16_round

_ORDER = ("x", "dt", "A_log", "B", "C", "h0")

# The workloads: the pages' Mamba 1 timing shapes (batch, inner width, length) at
# state width 16, bf16 I/O, one B/C group.
PCS_CONFIGS = {
    "pcs_balanced": dict(batch=16, channels=4096, seqlen=2048, dstate=16, ngroups=1, io="bf16", seed=20260011),
    "pcs_long": dict(batch=2, channels=2048, seqlen=32768, dstate=16, ngroups=1, io="bf16", seed=20260012),
}


def make_pcs_inputs(*, batch, channels, seqlen, dstate, ngroups=1, io="bf16", seed=0, init=False, dt_scale=1.0):
    """float32 arrays of storage-exact values: x, dt [b, L, D]; A_log [D, N];
    B, C [b, L, G, N]; h0 [b, D, N] (or None)."""
    ss = np.random.SeedSequence(seed)
    g = {k: np.random.Generator(np.random.PCG64(c)) for k, c in zip(_ORDER, ss.spawn(len(_ORDER)))}
    b, L, D, N, G = batch, seqlen, channels, dstate, ngroups
    rnd = (lambda a: bf16_round(a)) if io == "bf16" else (lambda a: np.asarray(a, np.float32))
    x = rnd(g["x"].standard_normal((b, L, D), dtype=np.float32))
    z = g["dt"].standard_normal((b, L, D), dtype=np.float32) * np.float32(0.5) - np.float32(2.0)
    dt = (np.logaddexp(np.float32(0.0), z) * np.float32(dt_scale)).astype(np.float32)
    A_log = np.log(g["A_log"].uniform(1.0, 16.0, size=(D, N))).astype(np.float32)
    B = rnd(g["B"].standard_normal((b, L, G, N), dtype=np.float32))
    C = rnd(g["C"].standard_normal((b, L, G, N), dtype=np.float32))
    h0 = (g["h0"].standard_normal((b, D, N), dtype=np.float32) * np.float32(0.1)) if init else None
    return {"x": x, "dt": dt, "A_log": A_log, "B": B, "C": C, "h0": h0}
