"""ctypes loader for the plain-C fp64 per-coordinate scan oracle (``pcs_cpu.c``).

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the
benchmark).  ``build()`` compiles the C file with gcc; ``scan()`` runs the
recurrence on all channels or a contiguous range of them.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pcs_cpu.c")
_LIB = os.path.join(_HERE, "libm3pcs.so")
_lib = None


def build(force=True):
    """Compile pcs_cpu.c into libm3pcs.so (gcc, -O2, OpenMP)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        I, P = ctypes.c_int, ctypes.c_void_p
        lib.m3ref_pcs.argtypes = [I] * 7 + [P] * 8 + [I]
        lib.m3ref_pcs.restype = I
        _lib = lib
    return _lib


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan(inp, h0=None, d0=0, d1=None, nthreads=0):
    """fp64 recurrence for channels [d0, d1) of every batch: returns
    (y [b, L, d1 - d0], h_final [b, d1 - d0, N])."""
    x, dt, A, B, C = (_f32(inp[k]) for k in ("x", "dt", "A_log", "B", "C"))
    b, L, D = x.shape
    G, N = B.shape[2], B.shape[3]
    d1 = D if d1 is None else d1
    y = np.zeros((b, L, d1 - d0))
    h1 = np.zeros((b, d1 - d0, N))
    h0 = _f32(h0)
    rc = _load().m3ref_pcs(b, L, D, G, N, d0, d1, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(h0), _p(y), _p(h1),
                           int(nthreads))
    if rc != 0:
        raise RuntimeError("m3ref_pcs failed (%d)" % rc)
    return y, h1
