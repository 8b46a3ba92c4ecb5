"""ctypes loader for the plain-C fp64 oracle (``ref_cpu.c``).

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the
benchmark).  ``build()`` compiles the C file with gcc; ``scan()`` runs the
sequential recurrence on all or on selected (batch, head) streams.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ref_cpu.c")
_LIB = os.path.join(_HERE, "libm3ref.so")
_lib = None


def build(force=True):
    """Compile ref_cpu.c into libm3ref.so (gcc, -O2, OpenMP)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.m3ref_scan.argtypes = [I] * 8 + [P] * 14 + [I, P, P] + [P] * 5 + [I]
        lib.m3ref_scan.restype = I
        lib.m3ref_max_threads.restype = I
        _lib = lib
    return _lib


def max_threads():
    return _load().m3ref_max_threads()


def _f32(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan(inp, sel=None, nthreads=0, want_y=True):
    """Run the fp64 recurrence.

    inp: dict from ``m3inputs.make_scan_inputs``.  sel: None for every stream
    (outputs in the full layouts y [b,L,H,R,P], h [b,H,P,N], ...), or a list
    of (batch, head) pairs (outputs stacked per stream: y [k,L,R,P], ...).
    """
    lib = _load()
    x = _f32(inp["x"])
    b, L, H, R, P = x.shape
    Bm, Cm = _f32(inp["B"]), _f32(inp["C"])
    G, N = Bm.shape[2], Bm.shape[4]
    th = _f32(inp.get("theta"))
    npairs = 0 if th is None else th.shape[3]
    init = inp.get("init") or {}
    keep = [x, Bm, Cm]
    args = {}
    for k in ("dt", "lam", "A_log", "A_raw", "B_bias", "C_bias"):
        args[k] = _f32(inp.get(k))
    ini = {k: _f32(init.get(k)) for k in ("h", "phi", "B_prev", "x_prev")}
    full = sel is None
    if full:
        sel = [(bi, h) for bi in range(b) for h in range(H)]
    sb = np.array([s[0] for s in sel], dtype=np.int32)
    sh = np.array([s[1] for s in sel], dtype=np.int32)
    k = len(sel)
    y = np.zeros((k, L, R, P)) if want_y else None
    hf = np.zeros((k, P, N))
    pf = np.zeros((k, npairs))
    bf = np.zeros((k, R, N))
    xf = np.zeros((k, R, P))
    rc = lib.m3ref_scan(b, L, H, G, P, N, R, npairs,
                        _ptr(x), _ptr(Bm), _ptr(Cm), _ptr(args["dt"]), _ptr(args["lam"]), _ptr(th),
                        _ptr(args["A_log"]), _ptr(args["A_raw"]), _ptr(args["B_bias"]), _ptr(args["C_bias"]),
                        _ptr(ini["h"]), _ptr(ini["phi"]), _ptr(ini["B_prev"]), _ptr(ini["x_prev"]),
                        k, _ptr(sb), _ptr(sh), _ptr(y), _ptr(hf), _ptr(pf), _ptr(bf), _ptr(xf),
                        int(nthreads))
    del keep
    if rc != 0:
        raise RuntimeError("m3ref_scan failed with status %d" % rc)
    fin = {"h": hf, "phi": pf, "B_prev": bf, "x_prev": xf}
    if full:
        if y is not None:
            y = y.reshape(b, H, L, R, P).transpose(0, 2, 1, 3, 4)
        fin = {kk: v.reshape((b, H) + v.shape[1:]) for kk, v in fin.items()}
    return y, fin
