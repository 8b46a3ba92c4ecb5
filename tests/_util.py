"""Helpers shared by the tests: moving seeded inputs to the device, error norms."""
import numpy as np
import torch


def rel_l2(a, b):
    """Normwise relative error ||a - b||_2 / ||b||_2 over the whole tensor."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def pooled_signed(a, b):
    """Pooled signed error sum(a - b) / ||b||_1 (a bias check)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.abs(b).sum()
    return float((a - b).sum() / (nb if nb > 0 else 1.0))


def tdev(a, dtype, dev):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev).to(dtype).contiguous()


def to_device(d, io_dtype, state_dtype, dev):
    """numpy input dict (m3inputs) -> torch tensors on ``dev``."""
    out = {}
    for k in ("x", "B", "C"):
        out[k] = tdev(d[k], io_dtype, dev)
    for k in ("dt", "lam", "theta", "A_log", "A_raw", "B_bias", "C_bias"):
        out[k] = tdev(d.get(k), torch.float32, dev)
    if d.get("init") is not None:
        i = d["init"]
        out["init"] = {"h": tdev(i["h"], state_dtype, dev), "phi": tdev(i["phi"], torch.float32, dev),
                       "B_prev": tdev(i["B_prev"], io_dtype, dev), "x_prev": tdev(i["x_prev"], io_dtype, dev)}
    else:
        out["init"] = None
    return out


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def phase_err(gpu_phi, ref_phi):
    """Phases compared through (cos, sin), so a wrap at 2 pi is no error."""
    g = np.asarray(gpu_phi, np.float64)
    r = np.asarray(ref_phi, np.float64)
    if g.size == 0:
        return 0.0
    return float(max(np.abs(np.cos(g) - np.cos(r)).max(), np.abs(np.sin(g) - np.sin(r)).max()))


ROW_TOL = 5e-2        # per-row bound for bf16 I/O (see row_errors)
ROW_FLOOR = 0.5       # denominator floor, as a fraction of the RMS row norm


def row_errors(g, r, floor_frac=None):
    """Per-row errors of one stream's outputs [L, R, P]: ||g - r|| over P, divided
    by max(||r||, ROW_FLOOR * the RMS row norm).  The floor keeps rows whose exact
    value nearly cancels from being judged by relative rounding noise; a wrong
    or dropped row still scores about 1."""
    floor_frac = ROW_FLOOR if floor_frac is None else floor_frac
    g = np.asarray(g, np.float64).reshape(-1, g.shape[-1])
    r = np.asarray(r, np.float64).reshape(-1, r.shape[-1])
    rn = np.linalg.norm(r, axis=1)
    floor = floor_frac * float(np.sqrt(np.mean(rn * rn))) if rn.size else 0.0
    return np.linalg.norm(g - r, axis=1) / np.maximum(rn, max(floor, 1e-30))
