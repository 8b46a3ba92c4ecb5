"""Seeded input generators (numpy).

Every tensor is drawn from ``numpy.random.Generator(PCG64(child))`` where the
children are spawned, in a fixed order, from ``SeedSequence(cfg.seed)``.
Values are rounded to the storage dtype here (bf16 by round-to-nearest-even),
so that the CPU oracle and the GPU receive bit-identical inputs: the oracle
upcasts the float32 values exactly, the GPU path takes the bf16 bit patterns.

Value laws (per workload text): x ~ N(0,1); B, C ~ N(0,1), optionally RMS-
normalised over the state axis (eps 1e-6) before rounding; dt =
softplus(N(-2, 0.5)); A_log = log U(1, 16) per head, or (per-token rates) a
rate input u ~ N(0, 1) per token; lambda = sigmoid(N(0,1))
or exactly 1; theta = U(0, pi) / N per rotating pair; bias ~ N(0, 0.1) (std);
h0 ~ N(0, 0.1).  These are input preparation only (the block's activations and
BCNorm sit outside the scan), not the scan's arithmetic.
"""
import math

import numpy as np

from .configs import Config

_ORDER = ("A_log", "dt", "lam", "theta", "x", "B", "C", "B_bias", "C_bias",
          "h0", "phi0", "B_prev0", "x_prev0", "A_raw")


def bf16_bits(a) -> np.ndarray:
    """uint16 bf16 bit patterns of ``a`` (float32 view), round-to-nearest-even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(a) -> np.ndarray:
    """float32 array whose values are exactly the bf16 (RNE) roundings of ``a``."""
    return bits_to_f32(bf16_bits(a))


def _round_io(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return bf16_round(a) if dtype == "bf16" else a


def _rngs(seed, spawn_key=()):
    ss = np.random.SeedSequence(seed, spawn_key=tuple(spawn_key))
    kids = ss.spawn(len(_ORDER))
    return {k: np.random.Generator(np.random.PCG64(c)) for k, c in zip(_ORDER, kids)}


def _normal(rng, shape, std=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _rms_normalise(a: np.ndarray) -> np.ndarray:
    ms = np.mean(np.square(a, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
    return a / np.sqrt(ms + np.float32(1e-6))


def make_scan_inputs(cfg: Config, seed=None, *, batch=None, seqlen=None, spawn_key=()):
    """All inputs of one scan call, as float32 arrays of storage-exact values.

    Returns a dict with x [b,L,H,R,P], B, C [b,L,G,R,N], dt, lam [b,L,H],
    theta [b,L,H,npairs] (None if npairs == 0), A_log [H], A_raw [b,L,H]
    (per-token rate inputs, None unless ``cfg.rate_dyn``), B_bias, C_bias
    [H,R,N] (None without bias) and init (None, or a dict h [b,H,P,N],
    phi [b,H,npairs], B_prev [b,H,R,N], x_prev [b,H,R,P]).
    """
    b = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    H, G, P, N, R, NP = cfg.nheads, cfg.ngroups, cfg.headdim, cfg.dstate, cfg.rank, cfg.npairs
    g = _rngs(cfg.seed if seed is None else seed, spawn_key)
    out = {}
    out["A_log"] = np.log(g["A_log"].uniform(1.0, 16.0, size=H)).astype(np.float32)
    out["A_raw"] = g["A_raw"].standard_normal((b, L, H)).astype(np.float32) if cfg.rate_dyn else None
    z = g["dt"].normal(-2.0, 0.5, size=(b, L, H))
    out["dt"] = np.logaddexp(0.0, z).astype(np.float32)          # softplus
    if cfg.lam_one:
        out["lam"] = np.ones((b, L, H), np.float32)
    else:
        out["lam"] = (1.0 / (1.0 + np.exp(-g["lam"].standard_normal((b, L, H))))).astype(np.float32)
    if NP > 0:
        out["theta"] = (g["theta"].uniform(0.0, math.pi, size=(b, L, H, NP)) / N).astype(np.float32)
    else:
        out["theta"] = None
    out["x"] = _round_io(_normal(g["x"], (b, L, H, R, P)), cfg.io_dtype)
    Bv = _normal(g["B"], (b, L, G, R, N))
    Cv = _normal(g["C"], (b, L, G, R, N))
    if cfg.rms_bc:
        Bv, Cv = _rms_normalise(Bv), _rms_normalise(Cv)
    out["B"] = _round_io(Bv, cfg.io_dtype)
    out["C"] = _round_io(Cv, cfg.io_dtype)
    if cfg.bias:
        out["B_bias"] = _normal(g["B_bias"], (H, R, N), 0.1)
        out["C_bias"] = _normal(g["C_bias"], (H, R, N), 0.1)
    else:
        out["B_bias"] = out["C_bias"] = None
    if cfg.init_state or cfg.init_full:
        h0 = _normal(g["h0"], (b, H, P, N), 0.1)
        h0 = _round_io(h0, cfg.state_dtype)
        init = {"h": h0,
                "phi": np.zeros((b, H, NP), np.float32),
                "B_prev": np.zeros((b, H, R, N), np.float32),
                "x_prev": np.zeros((b, H, R, P), np.float32)}
        if cfg.init_full:
            init["phi"] = g["phi0"].uniform(0.0, 2 * math.pi, size=(b, H, NP)).astype(np.float32)
            init["B_prev"] = _round_io(_normal(g["B_prev0"], (b, H, R, N)), cfg.io_dtype)
            init["x_prev"] = _round_io(_normal(g["x_prev0"], (b, H, R, P)), cfg.io_dtype)
        out["init"] = init
    else:
        out["init"] = None
    return out


def make_decode_inputs(cfg: Config, nsteps: int, seed=None, *, batch=None):
    """Inputs of ``nsteps`` decode steps, stacked on a time axis.

    Same layout as :func:`make_scan_inputs` with L = nsteps; step k uses
    index ``[:, k]`` of every per-token tensor.  The initial carry is always
    returned (zero unless the config draws one).
    """
    d = make_scan_inputs(cfg, seed, batch=batch, seqlen=nsteps, spawn_key=(7,))
    if d["init"] is None:
        b = cfg.batch if batch is None else batch
        H, P, N, R, NP = cfg.nheads, cfg.headdim, cfg.dstate, cfg.rank, cfg.npairs
        d["init"] = {"h": np.zeros((b, H, P, N), np.float32),
                     "phi": np.zeros((b, H, NP), np.float32),
                     "B_prev": np.zeros((b, H, R, N), np.float32),
                     "x_prev": np.zeros((b, H, R, P), np.float32)}
    return d


def make_small_case(seed, *, batch=1, seqlen=16, nheads=2, ngroups=None, headdim=4,
                    dstate=6, rank=2, npairs=2, chunk=4, io_dtype="f32",
                    state_dtype="f32", bias=True, lam_one=False, rms_bc=False,
                    init_full=True, dt_scale=1.0, rate_dyn=False):
    """A small random case for oracle self-tests and small GPU parity cases."""
    cfg = Config("small", batch=batch, seqlen=seqlen, nheads=nheads,
                 ngroups=nheads if ngroups is None else ngroups, headdim=headdim,
                 dstate=dstate, rank=rank, npairs=npairs, chunk=chunk,
                 io_dtype=io_dtype, state_dtype=state_dtype, bias=bias,
                 lam_one=lam_one, rms_bc=rms_bc, init_state=init_full,
                 init_full=init_full, rate_dyn=rate_dyn, seed_index=0)
    d = make_scan_inputs(cfg, seed=seed)
    if dt_scale != 1.0:
        d["dt"] = (d["dt"] * np.float32(dt_scale)).astype(np.float32)
    return cfg, d


_BLOCK_ORDER = ("z", "x", "B_raw", "C_raw", "dt_raw", "A_raw", "lam_raw", "th_raw",
                "dt_bias", "B_gain", "C_gain", "lift", "comb", "D", "B_bias", "C_bias", "init")


def make_block_inputs(cfg: Config, seed=None, *, batch=None, seqlen=None, init=True):
    """Inputs of one layer call (the steps around the scan), float32 arrays of
    storage-exact values.

    Raw projections: z, x [b,L,H,P] ~ N(0,1); B_raw, C_raw [b,L,G,R,N] ~ 2 N(0,1)
    (not normalised: the layer normalises them); dt_raw, A_raw, lam_raw [b,L,H] ~
    N(0,1) (dt_raw with std 0.5); th_raw [b,L,H,npairs] ~ N(0,1).  Parameters:
    dt_bias [H] ~ N(-3, 1) (steps of a few hundredths); B_gain,
    C_gain [N] ~ 1 + N(0, 0.1); lift, comb [H,R,P] ~ 1 + N(0, 0.1) (comb divided
    by R); D [H] ~ 1 + N(0, 0.1); B_bias, C_bias [H,R,N] ~ 1 + N(0, 0.1) (the
    biases start at ones).  init: a scan carry (x_prev is the lifted x) or None.
    The io tensors (z, x, B_raw, C_raw, and the carry's B_prev, x_prev) are
    rounded to the config's io dtype.
    """
    b = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    H, G, P, N, R, NP = cfg.nheads, cfg.ngroups, cfg.headdim, cfg.dstate, cfg.rank, cfg.npairs
    ss = np.random.SeedSequence(cfg.seed if seed is None else seed, spawn_key=(11,))
    g = {k: np.random.Generator(np.random.PCG64(c)) for k, c in zip(_BLOCK_ORDER, ss.spawn(len(_BLOCK_ORDER)))}
    io = cfg.io_dtype
    out = {"z": _round_io(_normal(g["z"], (b, L, H, P)), io),
           "x": _round_io(_normal(g["x"], (b, L, H, P)), io),
           "B_raw": _round_io(_normal(g["B_raw"], (b, L, G, R, N), 2.0), io),
           "C_raw": _round_io(_normal(g["C_raw"], (b, L, G, R, N), 2.0), io),
           "dt_raw": _normal(g["dt_raw"], (b, L, H), 0.5),
           "A_raw": _normal(g["A_raw"], (b, L, H)),
           "lam_raw": _normal(g["lam_raw"], (b, L, H)),
           "th_raw": _normal(g["th_raw"], (b, L, H, NP)) if NP > 0 else None}
    p = {"dt_bias": _normal(g["dt_bias"], (H,), 1.0) - np.float32(3.0),
         "B_gain": (1.0 + _normal(g["B_gain"], (N,), 0.1)).astype(np.float32),
         "C_gain": (1.0 + _normal(g["C_gain"], (N,), 0.1)).astype(np.float32),
         "lift": (1.0 + _normal(g["lift"], (H, R, P), 0.1)).astype(np.float32),
         "comb": ((1.0 + _normal(g["comb"], (H, R, P), 0.1)) / R).astype(np.float32),
         "D": (1.0 + _normal(g["D"], (H,), 0.1)).astype(np.float32),
         "B_bias": (1.0 + _normal(g["B_bias"], (H, R, N), 0.1)).astype(np.float32),
         "C_bias": (1.0 + _normal(g["C_bias"], (H, R, N), 0.1)).astype(np.float32)}
    out["params"] = p
    if init:
        gi = g["init"]
        out["init"] = {"h": _round_io(_normal(gi, (b, H, P, N), 0.1), cfg.state_dtype),
                       "phi": gi.uniform(0.0, 2 * math.pi, size=(b, H, NP)).astype(np.float32),
                       "B_prev": _round_io(_normal(gi, (b, H, R, N)), io),
                       "x_prev": _round_io(_normal(gi, (b, H, R, P)), io)}
    else:
        out["init"] = None
    return out


def make_cotangents(cfg: Config, seed=None, *, batch=None, seqlen=None, final=True):
    """Seeded output cotangents of one scan call (the backward pass's inputs):
    dy [b,L,H,R,P] ~ N(0,1) rounded to the I/O dtype, and (``final``) float32
    sensitivities of the final carry: h [b,H,P,N], phi [b,H,npairs],
    B_prev [b,H,R,N], x_prev [b,H,R,P], each ~ N(0,1) (None without ``final``)."""
    b = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    H, P, N, R, NP = cfg.nheads, cfg.headdim, cfg.dstate, cfg.rank, cfg.npairs
    ss = np.random.SeedSequence(cfg.seed if seed is None else seed, spawn_key=(13,))
    k = [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(5)]
    dy = _round_io(_normal(k[0], (b, L, H, R, P)), cfg.io_dtype)
    if not final:
        return dy, None
    dfin = {"h": _normal(k[1], (b, H, P, N)), "phi": _normal(k[2], (b, H, NP)),
            "B_prev": _normal(k[3], (b, H, R, N)), "x_prev": _normal(k[4], (b, H, R, P))}
    return dy, dfin
