"""CPU oracle of the Mamba-3 layer steps on either side of the scan: plain fp64 numpy.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module; the GPU library never
does, and it shares no code with the HIP kernels.

Sources (web pages, cited by title and section):

[M3]  "Mamba-3: Improved Sequence Modeling using State Space Principles"
      (intuitivepapers.ai explainer).
      - "Computing the rotation as a data-dependent RoPE", the decode listing:
        the step size is softplus of the raw step plus a per-head bias; the
        decay rate is the negated heavy-tail activation of its raw input; the
        trapezoid blend is sigmoid of its raw input; B and C are RMS-normalised
        and biased; each token adds dt * pi * tanh(raw angle) to the running
        angle; the output adds D times the input to the readout and is gated by
        silu(z).
      - "MIMO: a rank-4 state update for the same state size": x keeps the
        ordinary (P-wide) projection and is rescaled into R copies by a learned,
        data-independent vector (P R parameters per head).
      - "The Mamba-3 block, layer by layer": BCNorm is an RMSNorm on B and C
        right after the projection; the learned bias is added after the norm
        and before the rotation.
      - The remarks after the decode listing: the layer's nonlinearities are the
        softplus on the step, the sigmoid on lambda, the two RMSNorms, the SiLU
        on the gate and the heavy-tail rate activation; none acts on x.

Readings where the pages leave a step open (each is a reading, not a fact):
  * rms_norm(v) = g * v / sqrt(mean(v^2) + eps) over the state axis N, with one
    learned gain vector g [N] for B and one for C, shared by heads and ranks;
    eps = 1e-6.
  * The x lift is x_r = l[h, r] * x (elementwise, l [H, R, P]).
  * The pages do not say how the R readouts recombine; this oracle takes the
    mirror of the lift, y = sum_r w[h, r] * y_r (elementwise, w [H, R, P]).
  * The D skip adds D[h] times the un-lifted x; the gate multiplies the sum.
  * The scan between them is ``ref.scan_seq`` (heavy-tail rates) with the
    per-head biases applied inside it, exactly as in the scan-only path.
"""
import math

import numpy as np

from . import ref

RMS_EPS = 1e-6


def softplus(v):
    """log(1 + e^v), evaluated without overflow."""
    v = np.asarray(v, dtype=np.float64)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def sigmoid(v):
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * (1.0 + np.tanh(0.5 * v))


def silu(v):
    v = np.asarray(v, dtype=np.float64)
    return v * sigmoid(v)


def rms_norm(v, gain=None, eps=RMS_EPS):
    """[M3] "The Mamba-3 block": RMSNorm over the last axis, times a gain."""
    v = np.asarray(v, dtype=np.float64)
    out = v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    return out if gain is None else out * np.asarray(gain, dtype=np.float64)


def angle_rate(th_raw):
    """Per-token angular rate pi * tanh(raw): at most half a turn per unit step."""
    return math.pi * np.tanh(np.asarray(th_raw, dtype=np.float64))


def prologue(blk):
    """Raw projections -> the scan's inputs (fp64 arrays in the scan's layouts).

    blk keys: z, x [b,L,H,P]; B_raw, C_raw [b,L,G,R,N]; dt_raw, A_raw, lam_raw
    [b,L,H]; th_raw [b,L,H,np] or None; params dict with dt_bias [H], B_gain,
    C_gain [N] (or None), lift [H,R,P], comb [H,R,P], D [H] (or None), B_bias,
    C_bias [H,R,N] (or None); init (scan carry, lifted x_prev) or None.
    """
    p = blk["params"]
    f = lambda a: None if a is None else np.asarray(a, dtype=np.float64)  # noqa: E731
    x = f(blk["x"])
    lift = f(p["lift"])                                       # [H,R,P]
    xl = x[:, :, :, None, :] * lift[None, None]               # [b,L,H,R,P]
    dt = softplus(f(blk["dt_raw"]) + f(p["dt_bias"])[None, None, :])
    lam = sigmoid(f(blk["lam_raw"]))
    th = None if blk.get("th_raw") is None else angle_rate(blk["th_raw"])
    return {"x": xl, "B": rms_norm(blk["B_raw"], f(p.get("B_gain"))), "C": rms_norm(blk["C_raw"], f(p.get("C_gain"))),
            "dt": dt, "lam": lam, "theta": th, "A_log": None, "A_raw": f(blk["A_raw"]),
            "B_bias": f(p.get("B_bias")), "C_bias": f(p.get("C_bias")), "init": blk.get("init")}


def epilogue(blk, y):
    """Scan readouts y [b,L,H,R,P] -> layer output [b,L,H,P]: recombine the R
    readouts, add the D skip, gate by silu(z)."""
    p = blk["params"]
    comb = np.asarray(p["comb"], dtype=np.float64)            # [H,R,P]
    out = np.sum(np.asarray(y, dtype=np.float64) * comb[None, None], axis=3)
    if p.get("D") is not None:
        out = out + np.asarray(p["D"], dtype=np.float64)[None, None, :, None] * np.asarray(blk["x"], dtype=np.float64)
    return out * silu(blk["z"])


def block_forward(blk, scan=ref.scan_seq):
    """The layer between its input and output projections, whole sequence:
    (output [b,L,H,P], final scan carry)."""
    y, fin = scan(prologue(blk))
    return epilogue(blk, y), fin


def block_decode_step(carry, tok, params):
    """One token of the layer ([M3] decode listing, without the projections).

    tok keys: z, x [b,H,P]; B_raw, C_raw [b,G,R,N]; dt_raw, A_raw, lam_raw [b,H];
    th_raw [b,H,np] or None.  Returns (output [b,H,P], new carry).
    """
    one = {k: (None if v is None else np.asarray(v, dtype=np.float64)[:, None]) for k, v in tok.items()}
    one["params"] = params
    s = prologue(one)
    y, new = ref.decode_step(carry, s["x"][:, 0], s["B"][:, 0], s["C"][:, 0], s["dt"][:, 0], s["lam"][:, 0],
                             None if s["theta"] is None else s["theta"][:, 0], None,
                             s["B_bias"], s["C_bias"], A_raw=s["A_raw"][:, 0])
    return epilogue(one, y[:, None])[:, 0], new
