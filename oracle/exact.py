"""Exact rational brute force for tiny shapes (oracle side; test infrastructure).

Each fp16 input is converted exactly to a Fraction and every sum is formed
without rounding, so the results here are the mathematically exact values of
the definitions in ``reference`` -- the independent check that pins the
float64 oracle (pure-Python loops: keep shapes tiny).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _fr(v) -> Fraction:
    return Fraction(float(v))


def gemv_uniform_exact(x, codes, scales, zeros, g=128):
    M, K = x.shape
    N = codes.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                G = k // g
                acc += _fr(x[m, k]) * _fr(scales[n, G]) * (int(codes[n, k]) - int(zeros[n, G]))
            y[m][n] = acc
    return y


def gemv_lut4_exact(x, codes, absmax, lut, block=64):
    M, K = x.shape
    N = codes.shape[0]
    return [[sum((_fr(x[m, k]) * _fr(lut[int(codes[n, k])]) * _fr(absmax[n, k // block])
                  for k in range(K)), Fraction(0)) for n in range(N)] for m in range(M)]


def gemv_codebook_exact(x, codes, codebook, scales, g=128):
    M, K = x.shape
    N = codes.shape[0]
    v = codebook.shape[1]
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += _fr(x[m, k]) * _fr(scales[n, k // g]) * _fr(codebook[int(codes[n, k // v]), k % v])
            row.append(acc)
        out.append(row)
    return out


def gemv_codebook_additive_exact(x, codes, codebooks, scales, g):
    M, K = x.shape
    m, N, _ = codes.shape
    v = codebooks.shape[2]
    out = []
    for mm in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                c = sum((_fr(codebooks[i, int(codes[i, n, k // v]), k % v]) for i in range(m)), Fraction(0))
                acc += _fr(x[mm, k]) * _fr(scales[n, k // g]) * c
            row.append(acc)
        out.append(row)
    return out


def sparse_exact(x, N, rows, cols, vals):
    M = x.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    for r, c, v in zip(rows, cols, vals):
        for m in range(M):
            y[m][int(r)] += _fr(x[m, int(c)]) * _fr(v)
    return y


def gemv_dense_exact(x, w):
    M, K = x.shape
    return [[sum((_fr(x[m, k]) * _fr(w[n, k]) for k in range(K)), Fraction(0)) for n in range(w.shape[0])]
            for m in range(M)]


def to_f64(mat) -> np.ndarray:
    return np.array([[float(v) for v in row] for row in mat], dtype=np.float64)


def to_f16(mat) -> np.ndarray:
    """Round exact rationals to fp16: float64 first is exact here whenever the
    rational has <= 53 significant bits; callers keep shapes where that holds
    or accept the double-rounding caveat documented in the tests."""
    return to_f64(mat).astype(np.float16)
