"""Mamba-3 selective state-space scan for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``include/m3scan.h`` (``libm3scan.so``,
built in-tree by ``selective_state_space_mimo_amd.build``).  It only marshals
arguments: every step of the scan and of the decode step runs in the HIP
kernels of the library.  PyTorch supplies device memory and the current
stream.  There is no fallback: without the built library this package does
not import.

    y, final = scan_fwd(x, B, C, dt, lam, theta, A_log, B_bias, C_bias,
                        init=None, chunk=64)
    y = decode_step(x, B, C, dt, lam, theta, A_log, B_bias, C_bias, carry)
    grads = scan_bwd(x, B, C, dt, lam, theta, A_log, B_bias, C_bias, init, dy,
                     dfinal=None)

    y, h1 = pcs_fwd(x, dt, A_log, B, C, h0=None)     # per-coordinate scan

With ``A_raw=`` (a per-token rate input [b,L,H], or [b,H] for a decode step)
the decay rate of each token is the heavy-tail law (M3_RATE_HEAVY_TAIL) and
``A_log`` is not used.
"""
import ctypes
import os

import torch

__all__ = ["scan_fwd", "scan_fwd_noalloc", "scan_bwd", "decode_step", "scan_workspace_size", "new_carry", "M3Error",
           "pcs_fwd", "pcs_workspace_size", "pcs_desc", "PcsDesc",
           "LIB_PATH", "lib", "Desc", "Carry", "M3_F32", "M3_BF16", "M3_RATE_STATIC", "M3_RATE_HEAVY_TAIL"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libm3scan.so")
if not os.path.exists(LIB_PATH):
    raise ImportError("libm3scan.so is not built: run __graft_entry__.build() "
                      "(or python selective_state_space_mimo_amd/build.py)")

M3_F32, M3_BF16 = 0, 1
M3_RATE_STATIC, M3_RATE_HEAVY_TAIL = 0, 1
M3_ERR_TOO_LARGE = 5
_STATUS = {0: "M3_OK", 1: "M3_ERR_INVALID_ARG", 2: "M3_ERR_UNSUPPORTED", 3: "M3_ERR_ALIGNMENT", 4: "M3_ERR_HIP",
           5: "M3_ERR_TOO_LARGE"}


class Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int), ("seqlen", ctypes.c_int), ("nheads", ctypes.c_int),
                ("ngroups", ctypes.c_int), ("headdim", ctypes.c_int), ("dstate", ctypes.c_int),
                ("rank", ctypes.c_int), ("npairs", ctypes.c_int), ("chunk", ctypes.c_int),
                ("io_dtype", ctypes.c_int), ("state_dtype", ctypes.c_int), ("nsegments", ctypes.c_int),
                ("rate_law", ctypes.c_int)]


class Carry(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("phi", ctypes.c_void_p),
                ("B_prev", ctypes.c_void_p), ("x_prev", ctypes.c_void_p)]


lib = ctypes.CDLL(LIB_PATH)
_vp, _sz = ctypes.c_void_p, ctypes.c_size_t
lib.m3_scan_workspace_size.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(_sz)]
lib.m3_scan_workspace_size.restype = ctypes.c_int
lib.m3_scan_fwd.argtypes = [ctypes.POINTER(Desc)] + [_vp] * 9 + [ctypes.POINTER(Carry), _vp,
                                                               ctypes.POINTER(Carry), _vp, _sz, _vp]
lib.m3_scan_fwd.restype = ctypes.c_int
lib.m3_decode_step.argtypes = [ctypes.POINTER(Desc)] + [_vp] * 9 + [ctypes.POINTER(Carry), _vp, _vp]
lib.m3_decode_step.restype = ctypes.c_int
lib.m3_status_string.argtypes = [ctypes.c_int]
lib.m3_status_string.restype = ctypes.c_char_p
lib.m3_version.restype = ctypes.c_int


class M3Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = lib.m3_status_string(status).decode()
        super().__init__("%s: %s (%s)" % (where, _STATUS.get(status, status), msg))


def _check(st, where):
    if st != 0:
        raise M3Error(st, where)


def _dt(t):
    if t.dtype == torch.bfloat16:
        return M3_BF16
    if t.dtype == torch.float32:
        return M3_F32
    raise TypeError("unsupported dtype %s" % t.dtype)


def _ptr(t, dev, dtype=None, name=""):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device != dev:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, dev))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _carry(c, dev, io, st_dtype):
    if c is None:
        return None
    return Carry(_ptr(c["h"], dev, st_dtype, "h"), _ptr(c.get("phi"), dev, torch.float32, "phi"),
                 _ptr(c["B_prev"], dev, io, "B_prev"), _ptr(c["x_prev"], dev, io, "x_prev"))


def make_desc(x, B, theta, *, chunk=64, state_dtype=None, nsegments=0, decode=False, rate_law=M3_RATE_STATIC):
    if decode:
        b, H, R, P = x.shape
        G, N = B.shape[1], B.shape[3]
        L = 1
    else:
        b, L, H, R, P = x.shape
        G, N = B.shape[2], B.shape[4]
    npairs = 0 if theta is None else theta.shape[-1]
    sd = _dt(x) if state_dtype is None else (M3_BF16 if state_dtype == torch.bfloat16 else M3_F32)
    return Desc(b, L, H, G, P, N, R, npairs, chunk, _dt(x), sd, nsegments, rate_law)


def new_carry(batch, nheads, headdim, dstate, rank, npairs, io_dtype, state_dtype, device):
    """An all-zero carry dict (h, phi, B_prev, x_prev) on ``device``."""
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)  # noqa: E731
    return {"h": z((batch, nheads, headdim, dstate), state_dtype),
            "phi": z((batch, nheads, max(npairs, 0)), torch.float32),
            "B_prev": z((batch, nheads, rank, dstate), io_dtype),
            "x_prev": z((batch, nheads, rank, headdim), io_dtype)}


def scan_workspace_size(desc):
    n = _sz(0)
    _check(lib.m3_scan_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "m3_scan_workspace_size")
    return n.value


def scan_fwd(x, B, C, dt, lam, theta, A_log, B_bias=None, C_bias=None, init=None, *, chunk=64,
             state_dtype=torch.float32, nsegments=0, y=None, final=True, workspace=None, A_raw=None):
    """Chunked scan (``m3_scan_fwd``).

    x [b,L,H,R,P], B/C [b,L,G,R,N] (bf16 or f32, same dtype); dt, lam [b,L,H],
    theta [b,L,H,np] or None, A_log [H], biases [H,R,N] or None (all f32).
    init: None or dict(h [b,H,P,N] state_dtype, phi [b,H,np] f32, B_prev
    [b,H,R,N], x_prev [b,H,R,P]).  final: True to allocate and return the final
    carry, a dict to write into, or False/None to skip it.  A_raw: None for the
    static rates -exp(A_log), or the per-token rate input [b,L,H] f32 (the
    heavy-tail law; A_log is then ignored and may be None).
    Returns (y, final_carry_or_None).
    """
    dev = x.device
    io = x.dtype
    law = M3_RATE_STATIC if A_raw is None else M3_RATE_HEAVY_TAIL
    desc = make_desc(x, B, theta, chunk=chunk, state_dtype=state_dtype, nsegments=nsegments, rate_law=law)
    rate = A_log if A_raw is None else A_raw
    b, L, H, R, P = x.shape
    N = B.shape[4]
    if y is None:
        y = torch.empty_like(x)
    fin = None
    if final is True:
        fin = new_carry(b, H, P, N, R, desc.npairs, io, state_dtype, dev)
    elif isinstance(final, dict):
        fin = final
    ws_bytes = scan_workspace_size(desc)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ci, cf = _carry(init, dev, io, state_dtype), _carry(fin, dev, io, state_dtype)
    st = lib.m3_scan_fwd(ctypes.byref(desc), _ptr(x, dev, io, "x"), _ptr(B, dev, io, "B"), _ptr(C, dev, io, "C"),
                         _ptr(dt, dev, torch.float32, "dt"), _ptr(lam, dev, torch.float32, "lam"),
                         _ptr(theta, dev, torch.float32, "theta"), _ptr(rate, dev, torch.float32, "A_log/A_raw"),
                         _ptr(B_bias, dev, torch.float32, "B_bias"), _ptr(C_bias, dev, torch.float32, "C_bias"),
                         ctypes.byref(ci) if ci is not None else None, _ptr(y, dev, io, "y"),
                         ctypes.byref(cf) if cf is not None else None,
                         _ptr(workspace, dev, None, "workspace") if ws_bytes else None, ws_bytes, _stream(dev))
    _check(st, "m3_scan_fwd")
    return y, fin


lib.m3_scan_fwd_noalloc.argtypes = [ctypes.POINTER(Desc)] + [_vp] * 9 + [ctypes.POINTER(Carry), _vp,
                                                                       ctypes.POINTER(Carry), _vp]
lib.m3_scan_fwd_noalloc.restype = ctypes.c_int
lib.m3_scan_noalloc_max_workspace.argtypes = []
lib.m3_scan_noalloc_max_workspace.restype = _sz


def scan_fwd_noalloc(x, B, C, dt, lam, theta, A_log, B_bias=None, C_bias=None, init=None, *, y, final=None,
                     chunk=64, state_dtype=torch.float32, nsegments=0, A_raw=None):
    """Chunked scan without device allocation (``m3_scan_fwd_noalloc``): the
    caller passes the output ``y`` and, optionally, the final carry dict
    ``final``; the schedule's workspace is the library's per-GPU scratch.
    Arguments otherwise as for :func:`scan_fwd`.  Returns (y, final)."""
    dev = x.device
    io = x.dtype
    law = M3_RATE_STATIC if A_raw is None else M3_RATE_HEAVY_TAIL
    desc = make_desc(x, B, theta, chunk=chunk, state_dtype=state_dtype, nsegments=nsegments, rate_law=law)
    rate = A_log if A_raw is None else A_raw
    ci, cf = _carry(init, dev, io, state_dtype), _carry(final, dev, io, state_dtype)
    st = lib.m3_scan_fwd_noalloc(ctypes.byref(desc), _ptr(x, dev, io, "x"), _ptr(B, dev, io, "B"),
                                 _ptr(C, dev, io, "C"), _ptr(dt, dev, torch.float32, "dt"),
                                 _ptr(lam, dev, torch.float32, "lam"), _ptr(theta, dev, torch.float32, "theta"),
                                 _ptr(rate, dev, torch.float32, "A_log/A_raw"),
                                 _ptr(B_bias, dev, torch.float32, "B_bias"), _ptr(C_bias, dev, torch.float32, "C_bias"),
                                 ctypes.byref(ci) if ci is not None else None, _ptr(y, dev, io, "y"),
                                 ctypes.byref(cf) if cf is not None else None, _stream(dev))
    _check(st, "m3_scan_fwd_noalloc")
    return y, final


class PcsDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int), ("seqlen", ctypes.c_int), ("channels", ctypes.c_int),
                ("ngroups", ctypes.c_int), ("dstate", ctypes.c_int), ("io_dtype", ctypes.c_int),
                ("nsegments", ctypes.c_int)]


lib.m3_pcs_workspace_size.argtypes = [ctypes.POINTER(PcsDesc), ctypes.POINTER(_sz)]
lib.m3_pcs_workspace_size.restype = ctypes.c_int
lib.m3_pcs_fwd.argtypes = [ctypes.POINTER(PcsDesc)] + [_vp] * 8 + [_vp, _sz, _vp]
lib.m3_pcs_fwd.restype = ctypes.c_int


def pcs_desc(x, B, *, nsegments=0):
    b, L, D = x.shape
    G, N = B.shape[2], B.shape[3]
    return PcsDesc(b, L, D, G, N, _dt(x), nsegments)


def pcs_workspace_size(desc):
    n = _sz(0)
    _check(lib.m3_pcs_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "m3_pcs_workspace_size")
    return n.value


def pcs_fwd(x, dt, A_log, B, C, h0=None, *, y=None, h1=True, nsegments=0, workspace=None):
    """Per-coordinate selective scan, the Mamba 1 preset (``m3_pcs_fwd``).

    x [b,L,D], B/C [b,L,G,N] (bf16 or f32, same dtype); dt [b,L,D] and A_log
    [D,N] f32; h0 [b,D,N] f32 or None (zero).  h1: True to allocate and return
    the final state, a tensor to write into, or False/None to skip it.
    Returns (y, h1_or_None)."""
    dev = x.device
    io = x.dtype
    desc = pcs_desc(x, B, nsegments=nsegments)
    b, L, D = x.shape
    N = B.shape[3]
    if y is None:
        y = torch.empty_like(x)
    fin = None
    if h1 is True:
        fin = torch.empty((b, D, N), dtype=torch.float32, device=dev)
    elif isinstance(h1, torch.Tensor):
        fin = h1
    ws_bytes = pcs_workspace_size(desc)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = lib.m3_pcs_fwd(ctypes.byref(desc), _ptr(x, dev, io, "x"), _ptr(dt, dev, torch.float32, "dt"),
                        _ptr(A_log, dev, torch.float32, "A_log"), _ptr(B, dev, io, "B"), _ptr(C, dev, io, "C"),
                        _ptr(h0, dev, torch.float32, "h0"), _ptr(y, dev, io, "y"),
                        _ptr(fin, dev, torch.float32, "h1"),
                        _ptr(workspace, dev, None, "workspace") if ws_bytes else None, ws_bytes, _stream(dev))
    _check(st, "m3_pcs_fwd")
    return y, fin


class CarryGrad(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("phi", ctypes.c_void_p),
                ("B_prev", ctypes.c_void_p), ("x_prev", ctypes.c_void_p)]


class Grads(ctypes.Structure):
    _fields_ = [("dx", ctypes.c_void_p), ("dB", ctypes.c_void_p), ("dC", ctypes.c_void_p),
                ("ddt", ctypes.c_void_p), ("dlam", ctypes.c_void_p), ("dtheta", ctypes.c_void_p),
                ("dA", ctypes.c_void_p), ("dB_bias", ctypes.c_void_p), ("dC_bias", ctypes.c_void_p),
                ("dinit", CarryGrad)]


lib.m3_scan_bwd_workspace_size.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(_sz)]
lib.m3_scan_bwd_workspace_size.restype = ctypes.c_int
lib.m3_scan_bwd.argtypes = [ctypes.POINTER(Desc)] + [_vp] * 9 + [ctypes.POINTER(Carry), _vp, ctypes.POINTER(CarryGrad),
                                                               ctypes.POINTER(Grads), _vp, _sz, _vp]
lib.m3_scan_bwd.restype = ctypes.c_int


def scan_bwd_workspace_size(desc):
    n = _sz(0)
    _check(lib.m3_scan_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "m3_scan_bwd_workspace_size")
    return n.value


def _carry_grad(c, dev, name):
    if c is None:
        return CarryGrad(None, None, None, None)
    return CarryGrad(*[_ptr(c.get(k), dev, torch.float32, name + "." + k) for k in ("h", "phi", "B_prev", "x_prev")])


def scan_bwd(x, B, C, dt, lam, theta, A_log, B_bias, C_bias, init, dy, *, dfinal=None, state_dtype=torch.float32,
             A_raw=None, grads=None, want_init=True, workspace=None):
    """Gradients of the scan (``m3_scan_bwd``) for the loss sum(dy * y) plus the
    final carry's sensitivities ``dfinal`` (dict h, phi, B_prev, x_prev of float32
    tensors, any missing, or None).

    Forward inputs as for :func:`scan_fwd`.  Returns a dict: x, B, C (I/O dtype),
    dt, lam, theta (or None), A (d A_log [H], or d A_raw [b,L,H] with ``A_raw``),
    B_bias, C_bias (None without a bias), init (dict h, phi, B_prev, x_prev of
    float32, or None without ``want_init``).  ``grads`` may hold preallocated
    output tensors under the same keys."""
    dev = x.device
    io = x.dtype
    law = M3_RATE_STATIC if A_raw is None else M3_RATE_HEAVY_TAIL
    desc = make_desc(x, B, theta, state_dtype=state_dtype, rate_law=law)
    rate = A_log if A_raw is None else A_raw
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    npairs = desc.npairs
    f32 = torch.float32
    out = dict(grads or {})
    e = lambda k, shape, dt=f32: out[k] if out.get(k) is not None else torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
    out["x"] = e("x", x.shape, io)
    out["B"] = e("B", B.shape, io)
    out["C"] = e("C", C.shape, io)
    out["dt"] = e("dt", (b, L, H))
    out["lam"] = e("lam", (b, L, H))
    out["theta"] = e("theta", (b, L, H, npairs)) if npairs else None
    out["A"] = e("A", (b, L, H) if A_raw is not None else (H,))
    out["B_bias"] = e("B_bias", (H, R, N)) if B_bias is not None else None
    out["C_bias"] = e("C_bias", (H, R, N)) if C_bias is not None else None
    if want_init:
        di = dict(out.get("init") or {})
        out["init"] = {"h": di.get("h", torch.empty((b, H, P, N), dtype=f32, device=dev)),
                       "phi": di.get("phi", torch.empty((b, H, npairs), dtype=f32, device=dev)),
                       "B_prev": di.get("B_prev", torch.empty((b, H, R, N), dtype=f32, device=dev)),
                       "x_prev": di.get("x_prev", torch.empty((b, H, R, P), dtype=f32, device=dev))}
    else:
        out["init"] = None
    g = Grads(_ptr(out["x"], dev, io, "dx"), _ptr(out["B"], dev, io, "dB"), _ptr(out["C"], dev, io, "dC"),
              _ptr(out["dt"], dev, f32, "ddt"), _ptr(out["lam"], dev, f32, "dlam"),
              _ptr(out["theta"], dev, f32, "dtheta"), _ptr(out["A"], dev, f32, "dA"),
              _ptr(out["B_bias"], dev, f32, "dB_bias"), _ptr(out["C_bias"], dev, f32, "dC_bias"),
              _carry_grad(out["init"], dev, "dinit"))
    ws_bytes = scan_bwd_workspace_size(desc)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ci = _carry(init, dev, io, state_dtype)
    df = _carry_grad(dfinal, dev, "dfinal") if dfinal is not None else None
    st = lib.m3_scan_bwd(ctypes.byref(desc), _ptr(x, dev, io, "x"), _ptr(B, dev, io, "B"), _ptr(C, dev, io, "C"),
                         _ptr(dt, dev, f32, "dt"), _ptr(lam, dev, f32, "lam"), _ptr(theta, dev, f32, "theta"),
                         _ptr(rate, dev, f32, "A_log/A_raw"), _ptr(B_bias, dev, f32, "B_bias"),
                         _ptr(C_bias, dev, f32, "C_bias"), ctypes.byref(ci) if ci is not None else None,
                         _ptr(dy, dev, io, "dy"), ctypes.byref(df) if df is not None else None, ctypes.byref(g),
                         _ptr(workspace, dev, None, "workspace") if ws_bytes else None, ws_bytes, _stream(dev))
    _check(st, "m3_scan_bwd")
    return out


def decode_step(x, B, C, dt, lam, theta, A_log, B_bias, C_bias, carry, *, y=None, A_raw=None):
    """One decode step (``m3_decode_step``); ``carry`` (dict) is updated in place.

    x [b,H,R,P], B/C [b,G,R,N]; dt, lam [b,H]; theta [b,H,np] or None.
    Returns y [b,H,R,P]."""
    dev = x.device
    io = x.dtype
    law = M3_RATE_STATIC if A_raw is None else M3_RATE_HEAVY_TAIL
    desc = make_desc(x, B, theta, state_dtype=carry["h"].dtype, decode=True, rate_law=law)
    rate = A_log if A_raw is None else A_raw
    if y is None:
        y = torch.empty_like(x)
    c = _carry(carry, dev, io, carry["h"].dtype)
    st = lib.m3_decode_step(ctypes.byref(desc), _ptr(x, dev, io, "x"), _ptr(B, dev, io, "B"), _ptr(C, dev, io, "C"),
                            _ptr(dt, dev, torch.float32, "dt"), _ptr(lam, dev, torch.float32, "lam"),
                            _ptr(theta, dev, torch.float32, "theta"), _ptr(rate, dev, torch.float32, "A_log/A_raw"),
                            _ptr(B_bias, dev, torch.float32, "B_bias"), _ptr(C_bias, dev, torch.float32, "C_bias"),
                            ctypes.byref(c), _ptr(y, dev, io, "y"), _stream(dev))
    _check(st, "m3_decode_step")
    return y


# ---------------------------------------------------------------------------
# the layer steps around the scan (m3_block_fwd, m3_block_decode_step)
# ---------------------------------------------------------------------------
class BlockParams(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("B_gain", ctypes.c_void_p), ("C_gain", ctypes.c_void_p),
                ("B_bias", ctypes.c_void_p), ("C_bias", ctypes.c_void_p), ("lift", ctypes.c_void_p),
                ("comb", ctypes.c_void_p), ("D", ctypes.c_void_p), ("eps", ctypes.c_float)]


lib.m3_block_workspace_size.argtypes = [ctypes.POINTER(Desc), ctypes.c_int, ctypes.POINTER(_sz)]
lib.m3_block_workspace_size.restype = ctypes.c_int
lib.m3_block_fwd.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(BlockParams)] + [_vp] * 8 + [
    ctypes.POINTER(Carry), _vp, ctypes.POINTER(Carry), _vp, _sz, _vp]
lib.m3_block_fwd.restype = ctypes.c_int
lib.m3_block_decode_step.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(BlockParams)] + [_vp] * 8 + [
    ctypes.POINTER(Carry), _vp, _vp, _sz, _vp]
lib.m3_block_decode_step.restype = ctypes.c_int
__all__ += ["block_fwd", "block_decode_step", "block_workspace_size", "BlockParams"]


def _block_params(p, dev):
    f = lambda k: _ptr(p.get(k), dev, torch.float32, k)  # noqa: E731
    return BlockParams(f("dt_bias"), f("B_gain"), f("C_gain"), f("B_bias"), f("C_bias"), f("lift"), f("comb"),
                       f("D"), float(p.get("eps", 1e-6)))


def _block_desc(x, B_raw, R, th_raw, *, decode, chunk=64, state_dtype=None, nsegments=0, rate_law):
    if decode:
        b, H, P = x.shape
        G, N = B_raw.shape[1], B_raw.shape[3]
        L = 1
    else:
        b, L, H, P = x.shape
        G, N = B_raw.shape[2], B_raw.shape[4]
    npairs = 0 if th_raw is None else th_raw.shape[-1]
    sd = _dt(x) if state_dtype is None else (M3_BF16 if state_dtype == torch.bfloat16 else M3_F32)
    return Desc(b, L, H, G, P, N, R, npairs, chunk, _dt(x), sd, nsegments, rate_law)


def block_workspace_size(desc, decode=False):
    n = _sz(0)
    _check(lib.m3_block_workspace_size(ctypes.byref(desc), int(bool(decode)), ctypes.byref(n)),
           "m3_block_workspace_size")
    return n.value


def block_fwd(z, x, B_raw, C_raw, dt_raw, A, lam_raw, th_raw, params, init=None, *, chunk=64,
              state_dtype=torch.float32, nsegments=0, rate_law=M3_RATE_HEAVY_TAIL, out=None, final=True,
              workspace=None):
    """The layer steps around the scan over whole sequences (``m3_block_fwd``).

    z, x [b,L,H,P]; B_raw, C_raw [b,L,G,R,N] (bf16 or f32, same dtype); dt_raw,
    lam_raw [b,L,H] f32; A: the per-token rate input [b,L,H] (heavy-tail law) or
    A_log [H] with rate_law=M3_RATE_STATIC; th_raw [b,L,H,np] or None.  params:
    dict of f32 tensors lift, comb [H,R,P] (required), dt_bias [H], B_gain, C_gain
    [N], B_bias, C_bias [H,R,N], D [H] (each optional) and eps (float).
    Returns (out [b,L,H,P], final carry or None); the carry's x_prev holds the
    lifted x [b,H,R,P].
    """
    dev = x.device
    io = x.dtype
    R = B_raw.shape[3]
    desc = _block_desc(x, B_raw, R, th_raw, decode=False, chunk=chunk, state_dtype=state_dtype,
                       nsegments=nsegments, rate_law=rate_law)
    b, L, H, P = x.shape
    N = B_raw.shape[4]
    if out is None:
        out = torch.empty_like(x)
    fin = None
    if final is True:
        fin = new_carry(b, H, P, N, R, desc.npairs, io, state_dtype, dev)
    elif isinstance(final, dict):
        fin = final
    ws_bytes = block_workspace_size(desc)
    if ws_bytes and (workspace is None or workspace.numel() * workspace.element_size() < ws_bytes):
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    bp = _block_params(params, dev)
    ci, cf = _carry(init, dev, io, state_dtype), _carry(fin, dev, io, state_dtype)
    st = lib.m3_block_fwd(ctypes.byref(desc), ctypes.byref(bp), _ptr(z, dev, io, "z"), _ptr(x, dev, io, "x"),
                          _ptr(B_raw, dev, io, "B_raw"), _ptr(C_raw, dev, io, "C_raw"),
                          _ptr(dt_raw, dev, torch.float32, "dt_raw"), _ptr(A, dev, torch.float32, "A"),
                          _ptr(lam_raw, dev, torch.float32, "lam_raw"), _ptr(th_raw, dev, torch.float32, "th_raw"),
                          ctypes.byref(ci) if ci is not None else None, _ptr(out, dev, io, "out"),
                          ctypes.byref(cf) if cf is not None else None,
                          _ptr(workspace, dev, None, "workspace") if ws_bytes else None, ws_bytes, _stream(dev))
    _check(st, "m3_block_fwd")
    return out, fin


def block_decode_step(z, x, B_raw, C_raw, dt_raw, A, lam_raw, th_raw, params, carry, *,
                      rate_law=M3_RATE_HEAVY_TAIL, out=None, workspace=None):
    """One token of the layer (``m3_block_decode_step``); ``carry`` is updated in
    place.  z, x [b,H,P]; B_raw, C_raw [b,G,R,N]; dt_raw, lam_raw [b,H]; A [b,H]
    (or A_log [H] with rate_law=M3_RATE_STATIC); th_raw [b,H,np] or None.
    Returns out [b,H,P]."""
    dev = x.device
    io = x.dtype
    R = B_raw.shape[2]
    desc = _block_desc(x, B_raw, R, th_raw, decode=True, state_dtype=carry["h"].dtype, rate_law=rate_law)
    if out is None:
        out = torch.empty_like(x)
    ws_bytes = block_workspace_size(desc, decode=True)
    if workspace is None or workspace.numel() * workspace.element_size() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    bp = _block_params(params, dev)
    c = _carry(carry, dev, io, carry["h"].dtype)
    st = lib.m3_block_decode_step(ctypes.byref(desc), ctypes.byref(bp), _ptr(z, dev, io, "z"), _ptr(x, dev, io, "x"),
                                  _ptr(B_raw, dev, io, "B_raw"), _ptr(C_raw, dev, io, "C_raw"),
                                  _ptr(dt_raw, dev, torch.float32, "dt_raw"), _ptr(A, dev, torch.float32, "A"),
                                  _ptr(lam_raw, dev, torch.float32, "lam_raw"),
                                  _ptr(th_raw, dev, torch.float32, "th_raw"), ctypes.byref(c), _ptr(out, dev, io, "out"),
                                  _ptr(workspace, dev, None, "workspace"), ws_bytes, _stream(dev))
    _check(st, "m3_block_decode_step")
    return out
