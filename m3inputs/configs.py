"""The five workloads, as shapes and value laws.

Shapes follow the 1.5B-scale Mamba-3 layer described on "Mamba-3: Improved
Sequence Modeling using State Space Principles" (section "Why a recurrent
model's decode step is memory-bound": 64 heads of a 64 x 128 state, model
width 2,048 with expansion 2; section "MIMO: a rank-4 state update ...": R=4,
chunk 64 for the SISO kernels).  Value laws (softplus step, log-uniform decay
rate, sigmoid trapezoid weight, per-pair angular rate) follow the decode step
listing in section "Computing the rotation as a data-dependent RoPE".
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    seqlen: int          # tokens per sequence (scan); steps are separate for decode
    nheads: int
    ngroups: int         # B/C groups; head h reads group h * G // H
    headdim: int         # P
    dstate: int          # N
    rank: int            # R
    npairs: int          # rotating pairs (<= N/2); 0 = no rotation
    chunk: int           # Q (scan only)
    io_dtype: str        # "f32" | "bf16": x, B, C, y, B_prev, x_prev
    state_dtype: str     # "f32" | "bf16": h
    bias: bool           # per-head B/C bias [H,R,N] ~ N(0, 0.1)
    lam_one: bool        # lambda == 1 (no trapezoid term)
    rms_bc: bool         # B, C RMS-normalised over N before rounding
    init_state: bool     # h0 ~ N(0, 0.1); otherwise the carry starts at zero
    init_full: bool = False  # also random phi0 / B_prev0 / x_prev0 (tests only)
    decode_steps: int = 0    # > 0: a decode workload of that many steps
    rate_dyn: bool = False   # per-token decay rates (heavy-tail law of a rate input)
    seed_index: int = 0      # k in SeedSequence(20260000 + k)

    @property
    def seed(self) -> int:
        return 20260000 + self.seed_index

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = [
    Config("tiny_siso_f32", batch=1, seqlen=64, nheads=2, ngroups=2, headdim=16,
           dstate=16, rank=1, npairs=4, chunk=16, io_dtype="f32", state_dtype="f32",
           bias=False, lam_one=False, rms_bc=False, init_state=False, seed_index=1),
    Config("siso_bf16_mamba2", batch=4, seqlen=2048, nheads=32, ngroups=1, headdim=64,
           dstate=128, rank=1, npairs=0, chunk=64, io_dtype="bf16", state_dtype="f32",
           bias=False, lam_one=True, rms_bc=True, init_state=False, seed_index=2),
    Config("mimo_bf16_prefill", batch=8, seqlen=2048, nheads=64, ngroups=1, headdim=64,
           dstate=128, rank=4, npairs=32, chunk=64, io_dtype="bf16", state_dtype="f32",
           bias=True, lam_one=False, rms_bc=True, init_state=False, seed_index=3),
    Config("mimo_bf16_decode", batch=256, seqlen=1, nheads=64, ngroups=1, headdim=64,
           dstate=128, rank=4, npairs=32, chunk=64, io_dtype="bf16", state_dtype="bf16",
           bias=True, lam_one=False, rms_bc=True, init_state=True, decode_steps=1000,
           seed_index=4),
    Config("mimo_bf16_long", batch=1, seqlen=65536, nheads=64, ngroups=1, headdim=64,
           dstate=128, rank=4, npairs=32, chunk=128, io_dtype="bf16", state_dtype="f32",
           bias=True, lam_one=False, rms_bc=True, init_state=True, seed_index=5),
]


def config_by_name(name: str) -> Config:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)
