"""float64 reference results for every variant (oracle side; test infrastructure).

Every function takes the *logical* inputs (one code per byte, fp16 values as
numpy.float16), widens them exactly to float64 and returns ``(y_ref, A)``:

    y_ref[m, n] = sum_k x[m, k] * w[n, k]        (float64)
    A[m, n]     = sum_k |x[m, k] * w[n, k]|      (float64, the tolerance scale)

Accept a result y when ``|y - y_ref| <= 2e-3 * A + 1e-6``.  All products of
the inputs used here carry at most 11+8+11 significant bits, so each is exact
in float64; the only float64 error is the summation, below 1e-12 * A for
every shape in use.

Sources (titles of the pages; sections as the pages name them):

* Uniform group-wise asymmetric weights -- QFactory (ATC'25) review,
  "Problem and motivation" (low-bit, group-wise asymmetric scale/zero
  parameters) and "Experiments" (asymmetric W8/W4/W2, group 128x1).  The pages
  print no dequantization formula; reading taken: w = s * (q - z) with an
  integer zero point of the code's width.
* Zero-point algebraic expansion -- same page, "Key observations",
  observation 2 (paper sec. 4.3, Table 2): for one group it reduces to
  sum s(q - z)x = s(sum q x - z sum x).
* NF4-style lookup table -- "Fast NF4 Dequantization Kernels for Large
  Language Model Inference", abstract and method: 4-bit codes index 16
  normal-float levels, times a block-wise absmax scale (block 64 along K).
* Outlier-aware decomposition -- FlashQuant abstract: a low-bit dense path plus
  a high-precision sparse path sharing activations and outputs; the two add.
* Codebook / Psumbook -- CodeGEMM notes, "Key design 1" (Psumbook
  p_i^j = sum_k c_k^i x_k^j), "Overall framework" (build Psumbook -> read by
  code -> accumulate) and "Key design 4" (per-group normalization scale).
"""
from __future__ import annotations

import numpy as np

_ROW_CHUNK = 2048  # rows of W materialised at once


def _f64(a):
    return np.asarray(a).astype(np.float64)


def _gemv_rows(x64, wfun, N, rows=None):
    """Apply y = x W^T and A = |x| |W|^T over row chunks of W built by wfun(lo, hi)
    (or over the explicit row list `rows`)."""
    M = x64.shape[0]
    ax = np.abs(x64)
    if rows is None:
        y = np.empty((M, N))
        A = np.empty((M, N))
        for lo in range(0, N, _ROW_CHUNK):
            hi = min(N, lo + _ROW_CHUNK)
            w = wfun(np.arange(lo, hi))
            y[:, lo:hi] = x64 @ w.T
            A[:, lo:hi] = ax @ np.abs(w).T
        return y, A
    rows = np.asarray(rows, dtype=np.int64)
    w = wfun(rows)
    return x64 @ w.T, ax @ np.abs(w).T


def gemv_dense(x, w, rows=None):
    """y = x W^T for an fp16 weight W [N, K] used as given: the matrix product
    that follows an eager dequantization (Fast NF4 Dequantization Kernels page,
    method: the dequantized fp16 weight goes back to global memory for a
    separate product)."""
    w = np.asarray(w)
    return _gemv_rows(_f64(x), lambda r: _f64(w[r]), w.shape[0], rows)


# ----------------------------------------------------------------------------
# uniform W2 / W4 / W8
# ----------------------------------------------------------------------------

def dequant_uniform(codes, scales, zeros, g=128):
    """w[n, k] = s[n, k // g] * (q[n, k] - z[n, k // g])."""
    q = _f64(codes)
    s = np.repeat(_f64(scales), g, axis=1)
    z = np.repeat(_f64(zeros), g, axis=1)
    return s * (q - z)


def gemv_uniform(x, codes, scales, zeros, g=128, rows=None):
    x64 = _f64(x)

    def wfun(r):
        return dequant_uniform(codes[r], scales[r], zeros[r], g)

    return _gemv_rows(x64, wfun, codes.shape[0], rows)


def gemv_uniform_identity(x, codes, scales, zeros, g=128):
    """Same result through the group identity sum s(q-z)x = s(sum q x - z sum x)."""
    x64 = _f64(x)
    q = _f64(codes)
    s = _f64(scales)
    z = _f64(zeros)
    N, K = q.shape
    M = x64.shape[0]
    y = np.zeros((M, N))
    for G in range(K // g):
        xg = x64[:, G * g:(G + 1) * g]            # [M, g]
        qx = xg @ q[:, G * g:(G + 1) * g].T        # [M, N]  sum q x
        sx = xg.sum(axis=1, keepdims=True)         # [M, 1]  sum x
        y += s[:, G][None, :] * (qx - z[:, G][None, :] * sx)
    return y


# ----------------------------------------------------------------------------
# LUT4 (NF4-style)
# ----------------------------------------------------------------------------

def dequant_lut4(codes, absmax, lut, block=64):
    """w[n, k] = LUT[q[n, k]] * a[n, k // block]."""
    L = _f64(lut)
    return L[np.asarray(codes, dtype=np.int64)] * np.repeat(_f64(absmax), block, axis=1)


def quantize_activations_int8(x):
    """Symmetric per-row int8 activations (ADAngel review: arbitrary-precision
    quantization such as W4A8, activations at 8 bits; the pages fix no
    scheme, the plainest reading is one symmetric scale per row):
    s[m] = max_k |x[m, k]| / 127 and q[m, k] = rint(x[m, k] / s[m]) clamped to
    [-127, 127], both in float32 (the precision that decides the integers);
    a zero row gets s = 0 and q = 0."""
    x32 = np.asarray(x).astype(np.float32)
    amax = np.abs(x32).max(axis=1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint((x32 / safe[:, None]).astype(np.float32)).clip(-127, 127).astype(np.int8)
    return q, s


def gemv_w4a8(x, codes, scales, zeros, g=128, rows=None):
    """Padding strategy for W4A8 (ADAngel review, DPR: padding extends the
    low-bit weight to the activation width, here int4 codes to int8 (q - z)):
    y[m, n] = s_x[m] * sum_k s_w[n, k // g] * (q[n, k] - z[n, k // g]) * x_q[m, k].
    Tolerance scale: s_x[m] * sum_k |s_w (q - z) x_q|."""
    xq, sx = quantize_activations_int8(x)
    y, A = gemv_uniform(xq, codes, scales, zeros, g, rows=rows)
    sx64 = sx.astype(np.float64)[:, None]
    return y * sx64, A * sx64


def quantize_activations_asym8(x):
    """Asymmetric per-row int8 activations with an integer zero point, the
    activation side of a matmul whose two operands both carry zero points
    (QFactory review, observation 2: A_z1 . B_z2 expanded through all-ones J
    matrices).  The pages fix no activation scheme; reading taken: one fp32
    scale and one zero point per row mapping the row's range, widened to
    contain 0 (so that the zero point stays a signed byte), onto the signed
    byte range, every decision in fp32:
        lo, hi = min(min_k x, 0), max(max_k x, 0)
        s = (hi - lo) / 255,  zx = clamp(-128 - rint(lo / s), -128, 127)
        q = clamp(rint(x / s) + zx, -128, 127)
    (a zero row: s = 0, zx = 0, q = 0), and the activation the GEMV uses is
    s * (q - zx).  Returns (q int8 [M, K], s float32 [M], zx int32 [M])."""
    x32 = np.asarray(x).astype(np.float32)
    lo = np.minimum(x32.min(axis=1), np.float32(0.0))
    hi = np.maximum(x32.max(axis=1), np.float32(0.0))
    s = ((hi - lo).astype(np.float32) / np.float32(255.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    zx = np.where(s > 0, np.clip(-128.0 - np.rint((lo / safe).astype(np.float32)), -128, 127), 0).astype(np.int32)
    q = (np.rint((x32 / safe[:, None]).astype(np.float32)) + zx[:, None]).clip(-128, 127)
    q = np.where(s[:, None] > 0, q, 0).astype(np.int8)
    return q, s, zx


def gemv_w4a8_asym(x, codes, scales, zeros, g=128, rows=None):
    """W4A8 with asymmetric activations, by definition: both operands
    dequantized, y[m, n] = s_x[m] * sum_k s_w[n, k // g] (q[n, k] - z[n, k // g])
    (x_q[m, k] - zx[m]).  Tolerance scale: s_x[m] * sum_k |s_w (q - z) (x_q - zx)|."""
    xq, sx, zx = quantize_activations_asym8(x)
    xc = xq.astype(np.float64) - zx.astype(np.float64)[:, None]
    y, A = gemv_uniform(xc, codes, scales, zeros, g, rows=rows)
    sx64 = sx.astype(np.float64)[:, None]
    return y * sx64, A * sx64


def gemv_w4a8_asym_expanded(x, codes, scales, zeros, g=128):
    """The same result through the zero-point expansion of each group's
    integer dot product (QFactory review, observation 2, plain reading):
        sum_k (q - z)(x_q - zx) = sum_k q x_q - z sum_k x_q - zx sum_k q + g z zx
    with the raw codes and raw activation bytes, every term an exact integer."""
    xq, sx, zx = quantize_activations_asym8(x)
    q = np.asarray(codes).astype(np.int64)
    xi = xq.astype(np.int64)
    z = np.asarray(zeros).astype(np.int64)
    s = _f64(scales)
    N, K = q.shape
    M = xi.shape[0]
    y = np.zeros((M, N))
    for G in range(K // g):
        sl = slice(G * g, (G + 1) * g)
        qx = xi[:, sl] @ q[:, sl].T                      # [M, N] sum q x_q
        sx_ = xi[:, sl].sum(axis=1)[:, None]             # [M, 1] sum x_q
        sq = q[:, sl].sum(axis=1)[None, :]               # [1, N] sum q
        e = qx - z[:, G][None, :] * sx_ - zx[:, None].astype(np.int64) * sq + g * z[:, G][None, :] * zx[:, None]
        y += s[:, G][None, :] * e.astype(np.float64)
    return y * sx.astype(np.float64)[:, None]


def split_activations_int8(xq):
    """Split strategy's decomposition (ADAngel review, DPR: operands split by
    bits, partial products at a narrower width, outputs reconstructed): each
    int8 activation into a signed high nibble and an unsigned low nibble,
    x_q = 16 h + l with h in [-8, 7] and l in [0, 15]."""
    xi = np.asarray(xq).astype(np.int64)
    h = np.floor_divide(xi, 16)
    l = xi - 16 * h
    return h, l


def gemv_w4a8_split(x, codes, scales, zeros, g=128, rows=None):
    """W4A8 by the Split strategy: decomposition of the int8 activations
    into 4-bit slices (split_activations_int8), a partial product of each
    slice with the 4-bit weights (q - z), reconstruction
    P = 16 P_h + P_l per group, then the scales.  The same value as
    gemv_w4a8 (padding): the decomposition is exact."""
    xq, sx = quantize_activations_int8(x)
    h, l = split_activations_int8(xq)
    yh, Ah = gemv_uniform(h.astype(np.float64), codes, scales, zeros, g, rows=rows)
    yl, Al = gemv_uniform(l.astype(np.float64), codes, scales, zeros, g, rows=rows)
    sx64 = sx.astype(np.float64)[:, None]
    # tolerance scale: that of the reconstructed product
    _, A = gemv_uniform(xq.astype(np.float64), codes, scales, zeros, g, rows=rows)
    return (16.0 * yh + yl) * sx64, A * sx64


def gemv_lut4(x, codes, absmax, lut, block=64, rows=None):
    x64 = _f64(x)

    def wfun(r):
        return dequant_lut4(codes[r], absmax[r], lut, block)

    return _gemv_rows(x64, wfun, codes.shape[0], rows)


# ----------------------------------------------------------------------------
# outlier-aware W4 (dense + sparse fp16)
# ----------------------------------------------------------------------------

def sparse_part(x, N, o_rows, o_cols, o_vals):
    """S x^T for the COO outliers: y_s[m, r] += v * x[m, c]; also sum |v x|."""
    x64 = _f64(x)
    M = x64.shape[0]
    v = _f64(o_vals)
    ys = np.zeros((M, N))
    As = np.zeros((M, N))
    r = np.asarray(o_rows, dtype=np.int64)
    c = np.asarray(o_cols, dtype=np.int64)
    for m in range(M):
        np.add.at(ys[m], r, v * x64[m, c])
        np.add.at(As[m], r, np.abs(v * x64[m, c]))
    return ys, As


def add_sparse(y_prior, x, o_rows, o_cols, o_vals):
    """y_prior + S x^T: the separate sparse kernel of the unfused outlier
    pattern adds into the output the dense kernel already wrote (FlashQuant
    abstract: the two paths share activations and outputs).  The tolerance
    scale is |y_prior| + sum |v x|."""
    yp = _f64(y_prior)
    ys, As = sparse_part(x, yp.shape[1], o_rows, o_cols, o_vals)
    return yp + ys, np.abs(yp) + As


def gemv_outlier(x, codes, scales, zeros, o_rows, o_cols, o_vals, g=128, rows=None):
    """Dense codes are used as given (codes at outlier positions are not altered);
    the fp16 outliers are added on top."""
    yd, Ad = gemv_uniform(x, codes, scales, zeros, g, rows=rows)
    ys, As = sparse_part(x, codes.shape[0], o_rows, o_cols, o_vals)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        ys, As = ys[:, rows], As[:, rows]
    return yd + ys, Ad + As


# ----------------------------------------------------------------------------
# codebook (m = 1 codebook, v-dim centroids, per-group scale)
# ----------------------------------------------------------------------------

def dequant_codebook(codes, codebook, scales, g=128):
    """w[n, v*j + t] = s[n, (v*j + t) // g] * C[code[n, j], t]."""
    C = _f64(codebook)
    v = C.shape[1]
    cents = C[np.asarray(codes, dtype=np.int64)]          # [N, KC, v]
    N, KC = codes.shape
    w = cents.reshape(N, KC * v)
    return w * np.repeat(_f64(scales), g, axis=1)


def gemv_codebook(x, codes, codebook, scales, g=128, rows=None):
    x64 = _f64(x)

    def wfun(r):
        return dequant_codebook(codes[r], codebook, scales[r], g)

    return _gemv_rows(x64, wfun, codes.shape[0], rows)


def dequant_codebook_additive(codes, codebooks, scales, g):
    """m additive codebooks (CodeGEMM notes, "Key design 3": one kernel for any
    number of codebooks m, vector length v, code bits b and group g; the
    codebooks of a segment add up, as in the AQLM-style multi-codebook
    configurations the notes compare against):
    w[n, v*j + t] = s[n, (v*j + t) // g] * sum_i C_i[code_i[n, j], t]."""
    Cs = _f64(codebooks)                                   # [m, 256, v]
    codes = np.asarray(codes, dtype=np.int64)              # [m, N, KC]
    m, N, KC = codes.shape
    v = Cs.shape[2]
    cents = np.zeros((N, KC, v))
    for i in range(m):
        cents += Cs[i][codes[i]]
    return cents.reshape(N, KC * v) * np.repeat(_f64(scales), g, axis=1)


def gemv_codebook_additive(x, codes, codebooks, scales, g, rows=None):
    x64 = _f64(x)
    codes = np.asarray(codes)

    def wfun(r):
        return dequant_codebook_additive(codes[:, r], codebooks, scales[r], g)

    return _gemv_rows(x64, wfun, codes.shape[1], rows)


def psumbook(x, codebook):
    """P[m, j, c] = sum_t C[c, t] * x[m, v*j + t]  (one table per v-wide segment j)."""
    x64 = _f64(x)
    C = _f64(codebook)
    M, K = x64.shape
    v = C.shape[1]
    xs = x64.reshape(M, K // v, v)                        # [M, J, v]
    return xs @ C.T                                       # [M, J, ncent]


def gemv_codebook_psumbook(x, codes, codebook, scales, g=128):
    """Codebook-centric evaluation: build the Psumbook, read it by code,
    accumulate per group, scale per group."""
    P = psumbook(x, codebook)                             # [M, J, ncent]
    M, J, _ = P.shape
    v = np.asarray(codebook).shape[1]
    per_g = g // v
    codes = np.asarray(codes, dtype=np.int64)
    N = codes.shape[0]
    s = _f64(scales)
    y = np.zeros((M, N))
    jj = np.arange(J)
    for m in range(M):
        looked = P[m][jj[None, :], codes]                 # [N, J]
        grp = looked.reshape(N, J // per_g, per_g).sum(axis=2)
        y[m] = (grp * s).sum(axis=1)
    return y


# ----------------------------------------------------------------------------
# acceptance
# ----------------------------------------------------------------------------

def within_tolerance(y, y_ref, A, rel=2e-3, abs_=1e-6):
    """Boolean mask of |y - y_ref| <= rel*A + abs_ (y may be fp16 or float)."""
    y64 = _f64(y)
    return np.abs(y64 - y_ref) <= rel * A + abs_


def worst_ratio(y, y_ref, A, rel=2e-3, abs_=1e-6):
    """max over elements of |y - y_ref| / (rel*A + abs_) (<= 1 means pass)."""
    y64 = _f64(y)
    return float(np.max(np.abs(y64 - y_ref) / (rel * A + abs_))) if y64.size else 0.0
