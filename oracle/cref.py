"""ctypes binding of the plain C oracle ``cref.c`` (test infrastructure).

``build()`` compiles ``oracle/libqref.so`` with the host C compiler and
OpenMP; ``gemv_uniform`` runs it on the logical inputs (one code per byte,
fp16 values), packing them with this package's own bit-loop packer first.
Only tests and the CPU-baseline leg of the benchmark use it.
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

from . import formats

_DIR = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_DIR, "cref.c")
LIB = os.path.join(_DIR, "libqref.so")
_lib = None


def build() -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    tmp = LIB + ".tmp"
    subprocess.run([cc, "-O2", "-fPIC", "-shared", "-fopenmp", "-o", tmp, SRC, "-lm"], check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        L = ctypes.CDLL(LIB)
        vp, i = ctypes.c_void_p, ctypes.c_int
        L.qref_gemv_uniform.restype = i
        L.qref_gemv_uniform.argtypes = [i, i, i, i, i, vp, vp, vp, vp, i, i, vp, vp, i]
        L.qref_max_threads.restype = i
        _lib = L
    return _lib


def pack_inputs(codes, zeros, bits):
    """The plain packing of codes [N, K] and zero points [N, G] (bit loops)."""
    return formats.pack_plain(codes, bits), formats.pack_plain(zeros, bits)


def gemv_uniform(x, codes, scales, zeros, bits, g=128, rows=None, threads=0, packed=None):
    """(y_ref, A) in float64 over rows [row0, row1) (default: all), as
    ``reference.gemv_uniform``; ``packed`` = pack_inputs(...) to reuse."""
    x = np.ascontiguousarray(x, dtype=np.float16)
    s = np.ascontiguousarray(scales, dtype=np.float16)
    M, K = x.shape
    N = s.shape[0]
    qp, zp = packed if packed is not None else pack_inputs(codes, zeros, bits)
    qp = np.ascontiguousarray(qp, dtype=np.uint32)
    zp = np.ascontiguousarray(zp, dtype=np.uint32)
    r0, r1 = (0, N) if rows is None else rows
    y = np.empty((M, r1 - r0))
    A = np.empty((M, r1 - r0))
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    rc = lib().qref_gemv_uniform(bits, M, N, K, g, p(x.view(np.uint16)), p(qp), p(s.view(np.uint16)), p(zp),
                                 r0, r1, p(y), p(A), threads)
    if rc:
        raise ValueError(f"qref_gemv_uniform: bad arguments ({rc})")
    return y, A


def max_threads() -> int:
    return int(lib().qref_max_threads())
