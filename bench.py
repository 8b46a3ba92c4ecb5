#!/usr/bin/env python3
"""Benchmark of the Mamba-3 scan hot path on one MI355X.

Prints ONE JSON line.  ``value`` is the chunked scan's throughput in tokens/s
on the MIMO prefill workload (batch 8, 64 heads, P=64, N=128, R=4, L=2048,
chunk 64, bf16 I/O), timed over ``--steps`` calls after ``--warmup`` calls with
HIP events on the stream the kernels run on, inputs resident in HBM.  The same
line carries the decode step (batch 256, 64 heads, bf16 state, 1000 consecutive
steps) as GB/s against the 8 TB/s HBM peak, the other scan workloads, a
roofline object per kernel, and the CPU oracle timed on a bounded sample.

Algorithmic work (what the method must do; overheads are not credited):
  scan FLOP per head-token   R^2 (N + P)(Q + 1) + 4 R N P   (causal-trimmed chunked form)
  scan bytes per head-token  4 R P (x in, y out) + 4 R N G / H (B, C) + 8 (dt, lam) + 4 np (theta)
                             + per stream: final carry (state f32, phase, previous write)
  decode bytes per head-step 4 P N (bf16 state read + write) + 2 R P (x) + 4 R N G / H (B, C)
                             + 8 (dt, lam) + 4 np (theta) + 8 np (phase r/w) + 4 R N (B_prev r/w)
                             + 4 R P (x_prev r/w) + 2 R P (y)            = 37,288 B at R=4
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP32_VALU_TFLOPS = 157.3 # MI355X fp32 vector: 256 CUs x 4 SIMDs x 2.4 GHz x 64 flop (packed FMA)
CSRC = os.path.join(ROOT, "selective_state_space_mimo_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")
# sources that define each measured kernel (the counters stand only while these are unchanged)
KERNEL_SOURCES = {"scan": ("scan_mfma.hip", "scan_common.h", "m3_internal.h"), "decode": ("decode.hip", "m3_internal.h"),
                  "bwd": ("bwd.hip", "bwd_chunk.hip", "scan_common.h", "m3_internal.h"), "pcs": ("pcs.hip", "m3_internal.h"),
                  "layer": ("scan_mfma.hip", "scan_common.h", "m3_internal.h", "block.hip"),
                  "siso": ("scan_siso.hip", "scan_common.h", "m3_internal.h")}


def source_sha(kind):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kind, workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None when
    there is none or the kernel's sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    sha = source_sha(kind)
    for ln in lines:
        ln = ln.strip()
        if not ln.startswith("traffic:"):
            continue
        kv = dict(f.split("=", 1) for f in ln[len("traffic:"):].split() if "=" in f)
        if kv.get("kind") == kind and kv.get("workload") == workload and kv.get("source_sha256") == sha:
            return float(kv["bytes_per_launch"])
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default="scan3,decode4,scan2,scan5,scan3r,scan3q,layer3,bwd3,pcs,pcsl")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the 'copy' calibration workload")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic accounting
# ---------------------------------------------------------------------------
def executed_chunk(cfg):
    """Chunk length the library runs: the bf16 matrix-core path (P = 64, N = 128,
    R in {1, 2, 4}) holds at most 256 rows (tokens x ranks) per chunk and runs a
    longer request on the small-chunk schedule Q = 64 / R."""
    R, Q = cfg.rank, cfg.chunk
    if cfg.io_dtype == "bf16" and cfg.headdim == 64 and cfg.dstate == 128 and R in (1, 2, 4):
        return Q if Q * R <= 256 else 64 // R
    return Q


def scan_flops_per_head_token(cfg):
    """Matrix products of the chunked form per (head, token) at the executed chunk Q:
    scores and their application R^2 (N + P)(Q + 1) (the causal half of a Q x Q block,
    both products, 2 flops per multiply-add), state update and readout 4 R N P."""
    R, N, P, Q = cfg.rank, cfg.dstate, cfg.headdim, executed_chunk(cfg)
    return R * R * (N + P) * (Q + 1) + 4 * R * N * P


def scan_bytes(cfg, with_final=True):
    R, N, P, H, G, NP = cfg.rank, cfg.dstate, cfg.headdim, cfg.nheads, cfg.ngroups, cfg.npairs
    io = 2 if cfg.io_dtype == "bf16" else 4
    per_ht = 2 * io * R * P + 2 * io * R * N * G / H + 8 + 4 * NP + (4 if cfg.rate_dyn else 0)
    streams = cfg.batch * H
    total = per_ht * streams * cfg.seqlen
    if cfg.init_state:
        total += streams * P * N * 4
    if with_final:
        total += streams * (P * N * 4 + 4 * NP + io * R * (N + P))
    if cfg.bias:
        total += 2 * H * R * N * 4
    return total


BWD_CHUNK = 16     # tokens per chunk of the chunked (matrix-core) backward


def bwd_chunked(cfg):
    """Whether the library runs the backward in its chunked matrix-core form (bf16
    I/O, P 64, N 128, rank 4, at most 64 turning pairs)."""
    return (cfg.io_dtype == "bf16" and cfg.headdim == 64 and cfg.dstate == 128 and cfg.rank == 4
            and cfg.npairs <= 64)


def bwd_flops_per_head_token(cfg):
    """Matrix work per (head, token) of the backward.

    Chunked form (Q-token chunks, M = R Q rows): per chunk the score tiles
    S^T = Bt Ct^T and X dy^T (2 M^2 (N + P)), the weighted products dCt, dBt (2 M^2 N
    each) and dX (2 M^2 P), the state terms dy Hf_in, X Gf, Bt Gf^T and the carried
    sensitivity update (2 M P N each), and the forward pass's state update (2 M P N):
    2 R^2 Q (3 N + 2 P) + 10 R P N per head-token.

    Token-serial form: the readout's transpose dC = H^T dy (2 R P N), the sensitivity
    update G = alpha G + sum_r dy_r (x) C_r (2 R P N + P N), and v = G B, w = G^T X
    (2 R P N each); reconstructing the forward states is recomputation, not credited."""
    R, N, P = cfg.rank, cfg.dstate, cfg.headdim
    if bwd_chunked(cfg):
        return 2 * R * R * BWD_CHUNK * (3 * N + 2 * P) + 10 * R * P * N
    return 8 * R * P * N + P * N


def bwd_bytes(cfg):
    """Inputs read once (x, dy, B, C, dt, lambda, theta), gradients written once (dx,
    dB, dC, dt, lambda, theta), the initial and final carries and their sensitivities."""
    R, N, P, H, G, NP = cfg.rank, cfg.dstate, cfg.headdim, cfg.nheads, cfg.ngroups, cfg.npairs
    io = 2 if cfg.io_dtype == "bf16" else 4
    per_ht = 3 * io * R * P + 4 * io * R * N * G / H + 16 + 8 * NP + (8 if cfg.rate_dyn else 0)
    streams = cfg.batch * H
    total = per_ht * streams * cfg.seqlen
    total += streams * 2 * (P * N * 4 + 4 * NP + 4 * R * (N + P))   # final sensitivities in, initial gradients out
    if cfg.init_state:
        total += streams * P * N * 4
    if cfg.bias:
        total += 4 * H * R * N * 4
    return total


def decode_bytes_per_head_step(cfg):
    R, N, P, H, G, NP = cfg.rank, cfg.dstate, cfg.headdim, cfg.nheads, cfg.ngroups, cfg.npairs
    return 4 * P * N + 2 * R * P + 4 * R * N * G / H + 8 + 4 * NP + 8 * NP + 4 * R * N + 4 * R * P + 2 * R * P


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------
def time_calls(torch, fn, steps, warmup, ramp_s=0.25):
    """Mean ms per call over `steps` calls after `warmup`, HIP events on the
    current stream (the stream the library launches on).  Before the warm-up
    calls the workload runs untimed for `ramp_s` seconds: an idle GPU raises its
    clocks over the first tens of milliseconds of load, and a serving or training
    loop runs at the raised clocks."""
    t0 = time.time()
    while time.time() - t0 < ramp_s:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_launch_ms(torch, fn, n):
    """Mean ms of single calls, each bracketed by its own events (launch gaps excluded)."""
    s = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs]))


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
def run_scan(torch, m3, cfg, steps, warmup):
    from m3inputs import make_scan_inputs
    dev = torch.device("cuda:0")
    t0 = time.time()
    d = make_scan_inputs(cfg)
    io = torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32

    def T(a, dt):
        return None if a is None else torch.from_numpy(a).to(dev).to(dt).contiguous()
    x, B, C = T(d["x"], io), T(d["B"], io), T(d["C"], io)
    dt, lam, th, Al = T(d["dt"], torch.float32), T(d["lam"], torch.float32), T(d["theta"], torch.float32), \
        T(d["A_log"], torch.float32)
    Bb, Cb = T(d["B_bias"], torch.float32), T(d["C_bias"], torch.float32)
    Ar = T(d["A_raw"], torch.float32)
    init = None
    if d["init"] is not None:
        init = {"h": T(d["init"]["h"], torch.float32), "phi": T(d["init"]["phi"], torch.float32),
                "B_prev": T(d["init"]["B_prev"], io), "x_prev": T(d["init"]["x_prev"], io)}
    del d
    log("[bench] %s inputs ready in %.1fs" % (cfg.name, time.time() - t0))
    b, L, H, R, P = x.shape
    fin = m3.new_carry(b, H, P, cfg.dstate, R, cfg.npairs, io, torch.float32, dev)
    y = torch.empty_like(x)
    desc = m3.make_desc(x, B, th, chunk=cfg.chunk, state_dtype=torch.float32)
    ws_bytes = m3.scan_workspace_size(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def call():
        m3.scan_fwd(x, B, C, dt, lam, th, Al, Bb, Cb, init, chunk=cfg.chunk, y=y, final=fin, workspace=ws,
                    A_raw=Ar)
    ms = time_calls(torch, call, steps, warmup)
    ms_launch = per_launch_ms(torch, call, max(3, min(steps, 10)))
    toks = b * L
    flops = scan_flops_per_head_token(cfg) * b * L * H
    nbytes = scan_bytes(cfg)
    out = {"workload": cfg.name, "batch": b, "seqlen": L, "nheads": H, "headdim": P, "dstate": cfg.dstate,
           "rank": R, "chunk": cfg.chunk, "executed_chunk": executed_chunk(cfg), "npairs": cfg.npairs, "ngroups": cfg.ngroups,
           "ms_per_call": ms, "ms_per_launch": ms_launch, "tokens_per_s": toks / (ms * 1e-3),
           "algo_tflops": flops / (ms_launch * 1e-3) / 1e12, "algo_gbs": nbytes / (ms_launch * 1e-3) / 1e9,
           "flop_per_call": flops, "bytes_per_call": nbytes, "workspace_bytes": ws_bytes}
    out["mfma_frac"] = out["algo_tflops"] / PEAK_BF16_TFLOPS
    out["hbm_frac"] = out["algo_gbs"] / PEAK_HBM_GBS
    log("[bench] %s: %.3f ms/call, %.2f M tok/s, %.1f TFLOP/s (%.1f%% MFMA), %.0f GB/s (%.1f%% HBM)" % (
        cfg.name, ms, out["tokens_per_s"] / 1e6, out["algo_tflops"], 100 * out["mfma_frac"], out["algo_gbs"],
        100 * out["hbm_frac"]))
    del x, B, C, dt, lam, th, Ar, y, fin, init, ws
    torch.cuda.empty_cache()
    return out


# The per-coordinate scan (Mamba 1 preset).  Its work per coordinate-step (one
# channel, one token, one of the N state coordinates) is one exponential and four
# other fp32 VALU operations (the exponent dt a, the write dt x B, the decay
# multiply-add, the readout multiply-add).  A SIMD retires 32 fp32 lanes per cycle
# (the 157.3 TFLOP/s vector peak: 256 CUs x 4 SIMDs x 2.4 GHz x 32 lanes x 2 flop)
# and transcendentals at a quarter of that, 8 lanes per cycle, so a step costs
# 4 / 32 + 1 / 8 = 1 / 4 lane-cycle: the chip's ceiling is 256 x 4 x 2.4 GHz x 4 =
# 9830 G coordinate-steps/s.  HBM bytes per (channel, token): x and y in the I/O
# dtype, dt f32; B and C per (group, token); the states once per stream.
PCS_STEP_PEAK_G = 256 * 4 * 2.4 * 4
PCS_FLOP_PER_STEP = 6          # 2 products + 2 FMAs (the exponential counted apart)


def pcs_bytes(cfg):
    b, L, D, G, N = cfg["batch"], cfg["seqlen"], cfg["channels"], cfg["ngroups"], cfg["dstate"]
    io = 2 if cfg["io"] == "bf16" else 4
    return b * L * D * (2 * io + 4) + 2 * b * L * G * N * io + D * N * 4 + 2 * b * D * N * 4


def run_pcs(torch, m3, name, steps, warmup):
    from m3inputs.pcs import PCS_CONFIGS, make_pcs_inputs
    dev = torch.device("cuda:0")
    cfg = dict(PCS_CONFIGS[name])
    t0 = time.time()
    d = make_pcs_inputs(**{k: v for k, v in cfg.items()}, init=True)
    io = torch.bfloat16 if cfg["io"] == "bf16" else torch.float32

    def T(a, dt):
        return torch.from_numpy(a).to(dev).to(dt).contiguous()
    x, B, C = T(d["x"], io), T(d["B"], io), T(d["C"], io)
    dt, Al, h0 = T(d["dt"], torch.float32), T(d["A_log"], torch.float32), T(d["h0"], torch.float32)
    del d
    log("[bench] %s inputs ready in %.1fs" % (name, time.time() - t0))
    b, L, D = x.shape
    N = B.shape[3]
    y = torch.empty_like(x)
    h1 = torch.empty((b, D, N), dtype=torch.float32, device=dev)
    desc = m3.pcs_desc(x, B)
    ws_bytes = m3.pcs_workspace_size(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    def call():
        m3.pcs_fwd(x, dt, Al, B, C, h0, y=y, h1=h1, workspace=ws)
    ms = time_calls(torch, call, steps, warmup)
    ms_launch = per_launch_ms(torch, call, max(3, min(steps, 10)))
    steps_g = b * L * D * N / 1e9
    nbytes = pcs_bytes(cfg)
    out = {"workload": name, "batch": b, "seqlen": L, "channels": D, "dstate": N, "ngroups": cfg["ngroups"],
           "io": cfg["io"], "segments_workspace_bytes": ws_bytes, "ms_per_call": ms, "ms_per_launch": ms_launch,
           "tokens_per_s": b * L / (ms * 1e-3), "gsteps_per_s": steps_g / (ms_launch * 1e-3),
           "algo_gbs": nbytes / (ms_launch * 1e-3) / 1e9, "bytes_per_call": nbytes,
           "coordinate_steps_per_call": b * L * D * N}
    out["alu_frac"] = out["gsteps_per_s"] / PCS_STEP_PEAK_G
    out["hbm_frac"] = out["algo_gbs"] / PEAK_HBM_GBS
    out["valu_tflops"] = out["gsteps_per_s"] * PCS_FLOP_PER_STEP / 1e3
    log("[bench] %s: %.3f ms/call (%.3f ms/launch), %.2f M tok/s, %.0f Gstep/s (%.1f%% of the %.0f ALU "
        "ceiling), %.0f GB/s (%.1f%% HBM)" % (name, ms, ms_launch, out["tokens_per_s"] / 1e6, out["gsteps_per_s"],
                                             100 * out["alu_frac"], PCS_STEP_PEAK_G, out["algo_gbs"],
                                             100 * out["hbm_frac"]))
    del x, B, C, dt, Al, h0, y, h1, ws
    torch.cuda.empty_cache()
    return out


def pcs_cpu_baseline(name, budget_s):
    """The fp64 C oracle of the per-coordinate scan, as it stands, on a bounded
    sample: every batch and token of the first k channels."""
    from m3inputs.pcs import PCS_CONFIGS, make_pcs_inputs
    from oracle import pcs_cpu
    cfg = dict(PCS_CONFIGS[name])
    cores = cpu_cores()
    d = make_pcs_inputs(**cfg, init=True)
    D = cfg["channels"]
    t0 = time.time()
    pcs_cpu.scan(d, d["h0"], 0, 8, nthreads=cores)
    one = (time.time() - t0) / 8
    k = int(budget_s / max(one, 1e-5))
    k = max(cores, min(D, k - k % cores))
    t0 = time.time()
    pcs_cpu.scan(d, d["h0"], 0, k, nthreads=cores)
    dt = time.time() - t0
    toks = cfg["batch"] * cfg["seqlen"] * k / D          # whole tokens' worth of channels
    del d
    return {"value": toks / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%s: channels 0..%d of %d, every batch and token (%.2f%% of the workload) in %.1f s; fp64 "
                      "recurrence in C, channels over threads" % (name, k - 1, D, 100.0 * k / D, dt)}


def layer_bytes(cfg):
    """Algorithmic bytes of one layer call (the steps around the scan included):
    z, x and the output (P each per head-token), the raw B and C (shared by the
    heads of a group), the raw step, lambda and rate input, the raw angles, and the
    carries."""
    R, N, P, H, G, NP = cfg.rank, cfg.dstate, cfg.headdim, cfg.nheads, cfg.ngroups, cfg.npairs
    io = 2 if cfg.io_dtype == "bf16" else 4
    per_ht = 3 * io * P + 2 * io * R * N * G / H + 12 + 4 * NP
    streams = cfg.batch * H
    total = per_ht * streams * cfg.seqlen
    total += streams * (P * N * 4 + 4 * NP + io * R * (N + P)) * 2      # carry in and out
    return total


def run_layer(torch, m3, cfg, steps, warmup):
    """The layer entry point (m3_block_fwd) at a scan workload's shape."""
    from m3inputs import make_block_inputs
    dev = torch.device("cuda:0")
    d = make_block_inputs(cfg)
    io = torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32

    def T(a, dt):
        return None if a is None else torch.from_numpy(a).to(dev).to(dt).contiguous()
    t = {k: T(d[k], io) for k in ("z", "x", "B_raw", "C_raw")}
    for k in ("dt_raw", "A_raw", "lam_raw", "th_raw"):
        t[k] = T(d.get(k), torch.float32)
    params = {k: T(v, torch.float32) for k, v in d["params"].items()}
    params["eps"] = 1e-6
    init = {"h": T(d["init"]["h"], torch.float32), "phi": T(d["init"]["phi"], torch.float32),
            "B_prev": T(d["init"]["B_prev"], io), "x_prev": T(d["init"]["x_prev"], io)}
    del d
    b, L, H, P = t["x"].shape
    R = cfg.rank
    out = torch.empty_like(t["x"])
    fin = m3.new_carry(b, H, P, cfg.dstate, R, cfg.npairs, io, torch.float32, dev)
    ws = None

    def call():
        nonlocal ws
        _, _ = m3.block_fwd(t["z"], t["x"], t["B_raw"], t["C_raw"], t["dt_raw"], t["A_raw"], t["lam_raw"],
                            t["th_raw"], params, init, chunk=cfg.chunk, out=out, final=fin, workspace=ws)
    desc = m3._block_desc(t["x"], t["B_raw"], R, t["th_raw"], decode=False, chunk=cfg.chunk,
                          state_dtype=torch.float32, rate_law=m3.M3_RATE_HEAVY_TAIL)
    ws = torch.empty(max(m3.block_workspace_size(desc), 1), dtype=torch.uint8, device=dev)
    ms = time_calls(torch, call, steps, warmup)
    nbytes = layer_bytes(cfg)
    res = {"workload": cfg.name, "ms_per_call": ms, "tokens_per_s": b * L / (ms * 1e-3),
           "algo_gbs": nbytes / (ms * 1e-3) / 1e9, "bytes_per_call": nbytes,
           "workspace_bytes": int(ws.numel())}
    res["hbm_frac"] = res["algo_gbs"] / PEAK_HBM_GBS
    log("[bench] %s: %.3f ms/call, %.2f M tok/s, %.0f GB/s of layer I/O (%.1f%% HBM), workspace %.2f GB" % (
        cfg.name, ms, res["tokens_per_s"] / 1e6, res["algo_gbs"], 100 * res["hbm_frac"], ws.numel() / 1e9))
    del t, params, init, out, fin, ws
    torch.cuda.empty_cache()
    return res


def run_bwd(torch, m3, cfg, steps, warmup):
    """The backward pass (m3_scan_bwd) at a scan workload's shape, with output and
    final-carry sensitivities."""
    from m3inputs import make_cotangents, make_scan_inputs
    dev = torch.device("cuda:0")
    t0 = time.time()
    d = make_scan_inputs(cfg)
    dy, dfin = make_cotangents(cfg, seed=77)
    io = torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32

    def T(a, dt):
        return None if a is None else torch.from_numpy(a).to(dev).to(dt).contiguous()
    x, B, C = T(d["x"], io), T(d["B"], io), T(d["C"], io)
    dt, lam, th, Al = T(d["dt"], torch.float32), T(d["lam"], torch.float32), T(d["theta"], torch.float32), \
        T(d["A_log"], torch.float32)
    Bb, Cb = T(d["B_bias"], torch.float32), T(d["C_bias"], torch.float32)
    Ar = T(d["A_raw"], torch.float32)
    init = None
    if d["init"] is not None:
        init = {"h": T(d["init"]["h"], torch.float32), "phi": T(d["init"]["phi"], torch.float32),
                "B_prev": T(d["init"]["B_prev"], io), "x_prev": T(d["init"]["x_prev"], io)}
    dyt = T(dy, io)
    dft = {k: T(v, torch.float32) for k, v in dfin.items()}
    del d, dy, dfin
    log("[bench] %s backward inputs ready in %.1fs" % (cfg.name, time.time() - t0))
    b, L, H, R, P = x.shape
    desc = m3.make_desc(x, B, th, state_dtype=torch.float32,
                        rate_law=m3.M3_RATE_STATIC if Ar is None else m3.M3_RATE_HEAVY_TAIL)
    ws_bytes = m3.scan_bwd_workspace_size(desc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    grads = m3.scan_bwd(x, B, C, dt, lam, th, Al, Bb, Cb, init, dyt, dfinal=dft, A_raw=Ar, workspace=ws)

    def call():
        m3.scan_bwd(x, B, C, dt, lam, th, Al, Bb, Cb, init, dyt, dfinal=dft, A_raw=Ar, grads=grads, workspace=ws)
    ms = time_calls(torch, call, steps, warmup)
    ms_launch = per_launch_ms(torch, call, max(3, min(steps, 10)))
    flops = bwd_flops_per_head_token(cfg) * b * L * H
    nbytes = bwd_bytes(cfg)
    out = {"workload": cfg.name + "_backward", "batch": b, "seqlen": L, "nheads": H, "headdim": P,
           "dstate": cfg.dstate, "rank": R, "npairs": cfg.npairs, "ms_per_call": ms, "ms_per_launch": ms_launch,
           "tokens_per_s": b * L / (ms * 1e-3), "algo_tflops": flops / (ms_launch * 1e-3) / 1e12,
           "algo_gbs": nbytes / (ms_launch * 1e-3) / 1e9, "flop_per_call": flops, "bytes_per_call": nbytes,
           "workspace_bytes": ws_bytes}
    out["chunked"] = bwd_chunked(cfg)
    out["valu_frac"] = out["algo_tflops"] / PEAK_FP32_VALU_TFLOPS
    out["mfma_frac"] = out["algo_tflops"] / PEAK_BF16_TFLOPS
    out["hbm_frac"] = out["algo_gbs"] / PEAK_HBM_GBS
    peak = "%.1f%% of the bf16 MFMA peak" % (100 * out["mfma_frac"]) if out["chunked"] else \
        "%.1f%% of the fp32 VALU peak" % (100 * out["valu_frac"])
    log("[bench] %s: %.3f ms/call, %.2f M tok/s, %.1f TFLOP/s (%s), %.0f GB/s (%.1f%% HBM), workspace %.2f GB"
        % (out["workload"], ms, out["tokens_per_s"] / 1e6, out["algo_tflops"], peak, out["algo_gbs"],
           100 * out["hbm_frac"], ws_bytes / 1e9))
    del x, B, C, dt, lam, th, Ar, init, dyt, dft, grads, ws
    torch.cuda.empty_cache()
    return out


def run_decode(torch, m3, cfg, nsteps):
    dev = torch.device("cuda:0")
    t0 = time.time()
    from m3inputs.gen_torch import decode_inputs_device
    d = decode_inputs_device(cfg, nsteps, dev, cfg.seed)
    torch.cuda.synchronize()
    log("[bench] %s inputs (%d steps) ready in %.1fs" % (cfg.name, nsteps, time.time() - t0))
    b, H, R, P, N = cfg.batch, cfg.nheads, cfg.rank, cfg.headdim, cfg.dstate
    carry = m3.new_carry(b, H, P, N, R, cfg.npairs, torch.bfloat16, torch.bfloat16, dev)
    ys = torch.empty((b, H, R, P), dtype=torch.bfloat16, device=dev)

    def reset():
        carry["h"].copy_(d["h0"])
        for k in ("phi", "B_prev", "x_prev"):
            carry[k].zero_()

    def step(s):
        m3.decode_step(d["x"][s], d["B"][s], d["C"][s], d["dt"][s], d["lam"][s], d["theta"][s], d["A_log"],
                       d["B_bias"], d["C_bias"], carry, y=ys)
    # warm-up pass, then the timed 1000 consecutive steps from the seeded state
    reset()
    for s in range(min(nsteps, 20)):
        step(s)
    reset()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for s in range(nsteps):
        step(s)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / nsteps
    # per-launch duration (events around single steps)
    reset()
    ms_launch = per_launch_ms(torch, lambda: step(0), 50)
    per = decode_bytes_per_head_step(cfg)
    nbytes = per * b * H
    state_bytes = 4 * P * N * b * H
    out = {"workload": cfg.name, "batch": b, "nheads": H, "headdim": P, "dstate": N, "rank": R,
           "npairs": cfg.npairs, "steps": nsteps, "ms_per_step": ms, "ms_per_launch": ms_launch,
           "bytes_per_head_step": per, "bytes_per_step": nbytes,
           "gbs": nbytes / (ms_launch * 1e-3) / 1e9, "gbs_incl_gaps": nbytes / (ms * 1e-3) / 1e9,
           "state_gbs": state_bytes / (ms_launch * 1e-3) / 1e9}
    out["hbm_frac"] = out["gbs"] / PEAK_HBM_GBS
    log("[bench] %s: %.1f us/step (%.1f us/launch), %.0f GB/s (%.1f%% HBM), state-only %.0f GB/s" % (
        cfg.name, ms * 1e3, ms_launch * 1e3, out["gbs"], 100 * out["hbm_frac"], out["state_gbs"]))
    del d, carry
    torch.cuda.empty_cache()
    return out


def run_copy(torch, mib):
    """A plain device-to-device copy of a known size: the calibration kernel for
    the HBM byte counters (not part of the method)."""
    dev = torch.device("cuda:0")
    src = torch.empty(mib * (1 << 20) // 4, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)

    def call():
        dst.copy_(src)
    ms = time_calls(torch, call, 5, 2)
    nbytes = 2 * src.numel() * 4
    log("[bench] copy %d MiB: %.3f ms, %.0f GB/s (read + write)" % (mib, ms, nbytes / (ms * 1e-3) / 1e9))
    del src, dst
    torch.cuda.empty_cache()
    return {"workload": "copy", "bytes_read": mib << 20, "bytes_written": mib << 20, "ms_per_call": ms,
            "gbs": nbytes / (ms * 1e-3) / 1e9}


def cpu_cores():
    """Host threads this process may use (affinity, capped by OMP_NUM_THREADS)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return max(1, n)


def cpu_baseline(cfg, budget_s):
    """The fp64 C oracle, as it stands, on a bounded sample of the same scan
    workload: whole sequences of the first k (batch, head) streams, k chosen so
    that the timed run takes about ``budget_s`` seconds on the host cores."""
    from m3inputs import make_scan_inputs
    from oracle import ref_cpu
    cores = cpu_cores()
    d = make_scan_inputs(cfg)
    H, b = cfg.nheads, cfg.batch
    t0 = time.time()
    ref_cpu.scan(d, sel=[(0, 0)], nthreads=1, want_y=True)
    one = time.time() - t0                       # one stream, one thread
    k = int(budget_s * cores / max(one, 1e-4))
    k = max(1, min(b * H, k))
    if k >= cores:
        k -= k % cores                           # whole rounds of the thread pool
    sel = [(i // H, i % H) for i in range(k)]
    t0 = time.time()
    ref_cpu.scan(d, sel=sel, nthreads=cores, want_y=True)
    dt = time.time() - t0
    head_tokens = k * cfg.seqlen
    tok_s = head_tokens / dt / H                # a token is H head-tokens
    del d
    return {"value": tok_s, "unit": "tokens/s", "cores": min(cores, k), "kind": "oracle",
            "sample": "%s: the first %d of %d (batch, head) streams, full L=%d (%d head-tokens, %.2f%% of the "
                      "workload) in %.1f s; fp64 sequential recurrence in C, one stream per thread" % (
                cfg.name, k, b * H, cfg.seqlen, head_tokens, 100.0 * k / (b * H), dt)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only; the (batch, head) streams would shard across "
              "GPUs without communication, which is not built here. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import selective_state_space_mimo_amd as m3
    from m3inputs import config_by_name
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    wl = [w.strip() for w in args.workloads.split(",") if w.strip()]
    res = {}
    names = {"scan2": "siso_bf16_mamba2", "scan3": "mimo_bf16_prefill", "scan5": "mimo_bf16_long",
             "decode4": "mimo_bf16_decode", "scan3r": "mimo_bf16_prefill", "scan3q": "mimo_bf16_prefill",
             "layer3": "mimo_bf16_prefill", "bwd3": "mimo_bf16_prefill", "copy": None, "pcs": None,
             "pcsl": None}
    for w in wl:
        cfg = config_by_name(names[w]) if names[w] else None
        if w == "scan3r":      # the headline prefill with per-token heavy-tail rates
            cfg = cfg.with_(name="mimo_bf16_prefill_heavytail", rate_dyn=True)
        if w == "scan3q":      # the headline prefill on the small-chunk MIMO schedule (Q = 64 / R)
            cfg = cfg.with_(name="mimo_bf16_prefill_q16", chunk=64 // cfg.rank)
        if w == "layer3":      # the layer entry point (steps around the scan) at the prefill shape
            cfg = cfg.with_(name="mimo_bf16_layer")
        if w == "copy":
            res[w] = run_copy(torch, args.copy_mib)
        elif w.startswith("layer"):
            res[w] = run_layer(torch, m3, cfg, args.steps, args.warmup)
        elif w.startswith("bwd"):
            res[w] = run_bwd(torch, m3, cfg, max(3, args.steps // 2), args.warmup)
        elif w in ("pcs", "pcsl"):
            res[w] = run_pcs(torch, m3, "pcs_balanced" if w == "pcs" else "pcs_long", args.steps, args.warmup)
        elif w.startswith("scan"):
            steps = args.steps if w != "scan5" else max(3, args.steps // 4)
            res[w] = run_scan(torch, m3, cfg, steps, args.warmup)
        else:
            res[w] = run_decode(torch, m3, cfg, args.decode_steps)
    main_w = "scan3" if "scan3" in res else [w for w in wl if w != "copy"][0] if any(w != "copy" for w in wl) else "copy"
    if main_w in ("pcs", "pcsl"):
        main_w = "copy" if "copy" in res else main_w
    if main_w == "copy":
        print(json.dumps({"metric": "copy calibration", "value": res["copy"]["gbs"], "unit": "GB/s"}), flush=True)
        return
    prim = res[main_w]
    cpu = None
    if not args.no_cpu and main_w.startswith("scan"):
        cpu = cpu_baseline(config_by_name(names[main_w]), args.cpu_seconds)
        log("[bench] cpu oracle: %.1f tokens/s on %d cores (%s)" % (cpu["value"], cpu["cores"], cpu["sample"]))
    line = {
        "metric": "scan tokens/s (% MFMA peak) + decode state GB/s (% HBM peak), 1xMI355X",
        "value": prim.get("tokens_per_s", prim.get("gbs")),
        "unit": "tokens/s" if main_w.startswith(("scan", "pcs")) else "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": prim.get("ms_per_call", prim.get("ms_per_step")),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; shapes and value laws of the workloads)",
        "config": {"workload": prim["workload"], **{k: prim[k] for k in
                   ("batch", "seqlen", "nheads", "headdim", "dstate", "rank", "chunk", "npairs") if k in prim}},
    }
    if main_w.startswith("scan"):
        # the binding roof is the one whose floor (work / peak) is longer: at the headline
        # shape the arithmetic intensity (277 flop/B) sits just below the ridge (312 flop/B),
        # so the HBM roof binds; the MFMA fraction is reported beside it
        if prim["hbm_frac"] >= prim["mfma_frac"]:
            line["roofline"] = {"bound": "hbm", "achieved": prim["algo_gbs"], "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": prim["hbm_frac"],
                                "traffic": measured_traffic("scan", prim["workload"]),
                                "algorithmic_bytes": prim["bytes_per_call"],
                                "mfma_achieved_tflops": prim["algo_tflops"], "mfma_frac": prim["mfma_frac"],
                                "algorithmic_flops": prim["flop_per_call"]}
        else:
            line["roofline"] = {"bound": "mfma", "achieved": prim["algo_tflops"], "peak": PEAK_BF16_TFLOPS,
                                "unit": "TFLOP/s", "frac": prim["mfma_frac"],
                                "traffic": measured_traffic("scan", prim["workload"]),
                                "algorithmic_flops": prim["flop_per_call"], "algorithmic_bytes": prim["bytes_per_call"],
                                "hbm_achieved_gbs": prim["algo_gbs"], "hbm_frac": prim["hbm_frac"]}
    if "scan5" in res and main_w != "scan5":
        # the largest single-GPU scan (one sequence of 65536 tokens) with its own roofline
        lw = res["scan5"]
        bound = "hbm" if lw["hbm_frac"] >= lw["mfma_frac"] else "mfma"
        line["roofline_long"] = {"workload": lw["workload"], "bound": bound,
                                 "achieved": lw["algo_gbs"] if bound == "hbm" else lw["algo_tflops"],
                                 "peak": PEAK_HBM_GBS if bound == "hbm" else PEAK_BF16_TFLOPS,
                                 "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
                                 "frac": lw["hbm_frac"] if bound == "hbm" else lw["mfma_frac"],
                                 "traffic": measured_traffic("scan", lw["workload"]),
                                 "algorithmic_bytes": lw["bytes_per_call"], "algorithmic_flops": lw["flop_per_call"],
                                 "executed_chunk": lw["executed_chunk"], "ms_per_call": lw["ms_per_call"],
                                 "mfma_frac": lw["mfma_frac"], "hbm_frac": lw["hbm_frac"]}
    if "decode4" in res:
        dd = res["decode4"]
        line["decode"] = {"workload": dd["workload"], "gbs": dd["gbs"], "hbm_frac": dd["hbm_frac"],
                          "us_per_step": dd["ms_per_step"] * 1e3, "us_per_launch": dd["ms_per_launch"] * 1e3,
                          "state_gbs": dd["state_gbs"], "bytes_per_head_step": dd["bytes_per_head_step"]}
        line["roofline_decode"] = {"bound": "hbm", "achieved": dd["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": dd["hbm_frac"], "traffic": measured_traffic("decode", dd["workload"]),
                                   "algorithmic_bytes": dd["bytes_per_step"]}
    if "copy" in res:
        line["copy_calibration"] = res["copy"]
    layers = {k: v for k, v in res.items() if k.startswith("layer")}
    if layers:
        line["layer"] = {v["workload"]: {k2: v[k2] for k2 in ("tokens_per_s", "ms_per_call", "algo_gbs", "hbm_frac")}
                         for v in layers.values()}
    if "bwd3" in res:
        bw = res["bwd3"]
        line["backward"] = {k2: bw[k2] for k2 in ("workload", "tokens_per_s", "ms_per_call", "ms_per_launch",
                                                  "algo_tflops", "algo_gbs", "hbm_frac")}
        chunked = bw["chunked"]
        line["roofline_backward"] = {"bound": "mfma" if chunked else "alu", "achieved": bw["algo_tflops"],
                                     "peak": PEAK_BF16_TFLOPS if chunked else PEAK_FP32_VALU_TFLOPS,
                                     "unit": "TFLOP/s", "frac": bw["mfma_frac"] if chunked else bw["valu_frac"],
                                     "traffic": measured_traffic("bwd", bw["workload"]),
                                     "algorithmic_flops": bw["flop_per_call"],
                                     "algorithmic_bytes": bw["bytes_per_call"]}
    others = {k: v for k, v in res.items() if k != main_w and k.startswith("scan")}
    if others:
        line["scan_other"] = {v["workload"]: {"tokens_per_s": v["tokens_per_s"], "ms_per_call": v["ms_per_call"],
                                              "algo_tflops": v["algo_tflops"], "mfma_frac": v["mfma_frac"],
                                              "algo_gbs": v["algo_gbs"], "hbm_frac": v["hbm_frac"]}
                              for v in others.values()}
    pcs = {k: v for k, v in res.items() if k in ("pcs", "pcsl")}
    if pcs:
        line["pcs"] = {v["workload"]: {k2: v[k2] for k2 in ("tokens_per_s", "ms_per_call", "ms_per_launch",
                                                              "gsteps_per_s", "alu_frac", "algo_gbs", "hbm_frac",
                                                              "batch", "seqlen", "channels", "dstate")}
                       for v in pcs.values()}
        pw = pcs.get("pcs", next(iter(pcs.values())))
        line["roofline_pcs"] = {"bound": "alu", "achieved": pw["gsteps_per_s"], "peak": PCS_STEP_PEAK_G,
                                "unit": "Gstep/s", "frac": pw["alu_frac"], "workload": pw["workload"],
                                "traffic": measured_traffic("pcs", pw["workload"]),
                                "algorithmic_bytes": pw["bytes_per_call"],
                                "coordinate_steps": pw["coordinate_steps_per_call"],
                                "hbm_achieved_gbs": pw["algo_gbs"], "hbm_frac": pw["hbm_frac"]}
        if not args.no_cpu:
            line["cpu_baseline_pcs"] = pcs_cpu_baseline(pw["workload"], min(args.cpu_seconds, 8.0))
            log("[bench] pcs cpu oracle: %.1f tokens/s (%s)" % (line["cpu_baseline_pcs"]["value"],
                                                                 line["cpu_baseline_pcs"]["sample"]))
    line["cpu_baseline"] = cpu
    s = json.dumps(line)
    print(s, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(s + "\n")


if __name__ == "__main__":
    main()
