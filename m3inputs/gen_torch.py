"""Seeded decode-workload inputs drawn on the device (torch generator).

The 1000-step decode workload needs ~11 GB of per-step inputs; drawing them
with numpy on the host would take minutes, so they are drawn on the device
from a seeded torch generator with the same value laws as ``gen.py``
(x ~ N(0,1); B, C ~ N(0,1) RMS-normalised over N; dt = softplus(N(-2, 0.5));
lam = sigmoid(N(0,1)); theta = U(0, pi) / N; A_log = log U(1, 16); bias
~ N(0, 0.1); h0 ~ N(0, 0.1)), stored bf16 (round to nearest even).  Tests
hand the oracle copies of exactly these values.  No recurrence arithmetic.
"""
import math

import torch


def decode_inputs_device(cfg, nsteps, dev, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    b, H, G, R, P, N, NP = cfg.batch, cfg.nheads, cfg.ngroups, cfg.rank, cfg.headdim, cfg.dstate, cfg.npairs
    f32 = torch.float32
    x = torch.randn((nsteps, b, H, R, P), generator=g, device=dev, dtype=f32).to(torch.bfloat16)

    def bc():
        v = torch.randn((nsteps, b, G, R, N), generator=g, device=dev, dtype=f32)
        v = v * torch.rsqrt(v.square().mean(-1, keepdim=True) + 1e-6)
        return v.to(torch.bfloat16)
    B, C = bc(), bc()
    dt = torch.nn.functional.softplus(torch.randn((nsteps, b, H), generator=g, device=dev, dtype=f32) * 0.5 - 2.0)
    lam = torch.sigmoid(torch.randn((nsteps, b, H), generator=g, device=dev, dtype=f32))
    th = torch.rand((nsteps, b, H, NP), generator=g, device=dev, dtype=f32) * (math.pi / N)
    A_log = torch.log(torch.rand((H,), generator=g, device=dev, dtype=f32) * 15.0 + 1.0)
    Bb = torch.randn((H, R, N), generator=g, device=dev, dtype=f32) * 0.1
    Cb = torch.randn((H, R, N), generator=g, device=dev, dtype=f32) * 0.1
    h0 = (torch.randn((b, H, P, N), generator=g, device=dev, dtype=f32) * 0.1).to(torch.bfloat16)
    return dict(x=x, B=B, C=C, dt=dt, lam=lam, theta=th, A_log=A_log, B_bias=Bb, C_bias=Cb, h0=h0)


def stream_inputs_host(d, bi, h, G=1, H=None):
    """numpy scan inputs of one (batch, head) stream of a device decode
    workload, laid out as a scan over the steps (batch 1, one head)."""
    import numpy as np
    H = d["x"].shape[2] if H is None else H
    g = h * G // H
    f = lambda t: t.float().cpu().numpy().astype(np.float32)  # noqa: E731
    S = d["x"].shape[0]
    out = {
        "x": f(d["x"][:, bi, h])[None, :, None],                 # [1,S,1,R,P]
        "B": f(d["B"][:, bi, g])[None, :, None],                 # [1,S,1,R,N]
        "C": f(d["C"][:, bi, g])[None, :, None],
        "dt": f(d["dt"][:, bi, h]).reshape(1, S, 1),
        "lam": f(d["lam"][:, bi, h]).reshape(1, S, 1),
        "theta": f(d["theta"][:, bi, h])[None, :, None] if d["theta"].shape[-1] else None,
        "A_log": f(d["A_log"][h:h + 1]),
        "B_bias": f(d["B_bias"][h:h + 1]),
        "C_bias": f(d["C_bias"][h:h + 1]),
    }
    R, N = d["B"].shape[3], d["B"].shape[4]
    P = d["x"].shape[4]
    NP = d["theta"].shape[-1]
    out["init"] = {"h": f(d["h0"][bi, h])[None, None], "phi": np.zeros((1, 1, NP), np.float32),
                   "B_prev": np.zeros((1, 1, R, N), np.float32), "x_prev": np.zeros((1, 1, R, P), np.float32)}
    return out
