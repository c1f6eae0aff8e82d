"""Python binding of libqgemv.so (fused dequantize-and-multiply GEMV, MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  torch supplies device memory and the current stream.
There is no fallback: if the library is missing, every call raises.

The C ABI is declared in ``include/qgemv.h``; function names here mirror it.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqgemv.so")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_VALUE, ERR_HIP = range(8)
PATH_AUTO, PATH_VALU, PATH_MFMA = 0, 1, 2
LAYOUT_PLAIN, LAYOUT_DEVICE, LAYOUT_ROWS64 = 0, 1, 2
GROUP = 128
# qgemv_variant (weight formats, for workspace_bytes)
W2, W4, W8, LUT4, OUTLIER4, CODEBOOK, W4A8, W4A8_SPLIT, W4A8_ASYM = 2, 4, 8, 16, 17, 18, 19, 20, 21
LAYOUT_VERSION = 1  # QGEMV_LAYOUT_VERSION of the header this binding follows

_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_i64 = ctypes.c_int64

# name -> (restype, argtypes); kept in step with include/qgemv.h
_SIGS = {
    "qgemv_version": (_i, []),
    "qgemv_layout_version": (_i, []),
    "qgemv_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "qgemv_status_string": (ctypes.c_char_p, [_i]),
    "qgemv_last_hip_error": (_i, []),
    "qgemv_packed_words": (_sz, [_i, _i, _i, _i]),
    "qgemv_pack": (_i, [_i, _i, _i, _i, _vp, _vp, _vp]),
    "qgemv_unpack": (_i, [_i, _i, _i, _i, _vp, _vp, _vp]),
    "qgemv_w2a16": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "qgemv_w4a16": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "qgemv_w8a16": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "qgemv_uniform": (_i, [_i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "qgemv_lut4": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "qgemv_outlier": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int64, _vp, _vp]),
    "qgemv_tilecoo_ptr_len": (_sz, [_i, _i]),
    "qgemv_codebook": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "qgemv_codebook_workspace_bytes": (_sz, [_i, _i, _i]),
    "qgemv_tilecoo_encode": (_i, [_i, _i, ctypes.c_int64, _vp, _vp, _vp, _vp, _vp]),
    "qgemv_w4a8": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "qgemv_w4a8_workspace_bytes": (_sz, [_i, _i]),
    "qgemv_w4a8_noalloc": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "qgemv_w4a8_split": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "qgemv_w4a8_split_workspace_bytes": (_sz, [_i, _i]),
    "qgemv_w4a8_asym": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "qgemv_w4a8_asym_workspace_bytes": (_sz, [_i, _i]),
    "qgemv_stream_read": (_i, [_vp, _sz, _vp, _i, _i, _vp]),
    "qgemv_gemm_uniform": (_i, [_i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp]),
    "qgemv_codebook_gen": (_i, [_i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "qgemv_codebook_gen_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "qgemv_dequant": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "qgemv_dequant_lut4": (_i, [_i, _i, _vp, _vp, _vp, _vp, _vp]),
    "qgemv_gemv_f16": (_i, [_i, _i, _i, _vp, _vp, _vp, _vp]),
    "qgemv_spmv_tilecoo": (_i, [_i, _i, _i, _vp, _vp, _vp, ctypes.c_int64, _vp, _vp]),
}


class QgemvError(RuntimeError):
    def __init__(self, fn, status):
        msg = lib().qgemv_status_string(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError {lib().qgemv_last_hip_error()})"
        super().__init__(f"{fn}: {msg} [{status}]")
        self.status = status


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m gemm_unpack_bit_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn, status):
    if status != OK:
        raise QgemvError(fn, status)


# ----------------------------------------------------------------------------
# torch marshalling
# ----------------------------------------------------------------------------

def _torch():
    import torch

    return torch


def _ptr(t):
    return _vp(t.data_ptr()) if t is not None else _vp(0)


def _stream(t):
    torch = _torch()
    return _vp(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def layout_version():
    """Version of the packed formats (packed buffers are valid only for a
    library reporting the same one)."""
    return int(lib().qgemv_layout_version())


def workspace_bytes(variant, M, N, K):
    """Scratch bytes the compute call of `variant` (W2 .. W4A8) needs at (M, N, K)."""
    return int(lib().qgemv_workspace_bytes(variant, M, N, K))


def packed_words(bits, rows, cols, layout=LAYOUT_DEVICE):
    return int(lib().qgemv_packed_words(bits, layout, rows, cols))


def pack(codes, bits, layout=LAYOUT_DEVICE):
    """[R, C] uint8 codes (one per byte) -> int32 words: [R, ceil(C*b/32)] for the
    plain layout, flat [packed_words] for the tiled device layout."""
    torch = _torch()
    _need(codes, torch.uint8, "codes")
    R, C = codes.shape
    n = packed_words(bits, R, C, layout)
    if n == 0 and R and C:
        raise ValueError("bad bits/shape for this layout")
    shape = (R, n // R if R else 0) if layout == LAYOUT_PLAIN else (n,)
    out = torch.empty(shape, dtype=torch.int32, device=codes.device)
    _check("qgemv_pack", lib().qgemv_pack(bits, layout, R, C, _ptr(codes), _ptr(out), _stream(codes)))
    return out


def unpack(packed, bits, rows, cols, layout=LAYOUT_DEVICE):
    torch = _torch()
    _need(packed, torch.int32, "packed")
    R = rows
    out = torch.empty((R, cols), dtype=torch.uint8, device=packed.device)
    _check("qgemv_unpack", lib().qgemv_unpack(bits, layout, R, cols, _ptr(packed), _ptr(out), _stream(packed)))
    return out


def pack_zeros(zeros, bits):
    """[N, G] uint8 zero points -> plain-packed int32 words (the zero-point format)."""
    return pack(zeros, bits, LAYOUT_PLAIN)


def uniform(x, wq, scales, zeros, bits, path=PATH_AUTO, out=None):
    """y = x . dequant(Wq)^T for group-wise asymmetric b-bit weights.

    x [M, K] fp16; wq int32 words in the device layout; scales [N, K/128] fp16;
    zeros [N, ceil(K/128*b/32)] int32 (plain packed).  Returns y [M, N] fp16."""
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(wq, torch.int32, "wq")
    _need(scales, torch.float16, "scales")
    _need(zeros, torch.int32, "zeros")
    M, K = x.shape
    N = scales.shape[0]
    need = packed_words(bits, N, K)  # 0 for bits/K the library rejects itself
    if need and wq.numel() != need:
        raise ValueError("wq does not hold N x K device-layout codes")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out")
    _check("qgemv_uniform", lib().qgemv_uniform(bits, path, M, N, K, _ptr(x), _ptr(wq), _ptr(scales),
                                                _ptr(zeros), _ptr(out), _stream(x)))
    return out


def w2a16(x, wq, scales, zeros, out=None):
    return uniform(x, wq, scales, zeros, 2, PATH_AUTO, out)


def w4a16(x, wq, scales, zeros, out=None):
    return uniform(x, wq, scales, zeros, 4, PATH_AUTO, out)


def w8a16(x, wq, scales, zeros, out=None):
    return uniform(x, wq, scales, zeros, 8, PATH_AUTO, out)


def lut4(x, wq, absmax, lut, out=None):
    """y = x . (lut[q] * absmax)^T for 4-bit codes with a 16-entry fp16 table.

    x [M, K] fp16; wq int32 4-bit codes in the device layout; absmax [N, K/64]
    fp16 (one scale per 64 consecutive k); lut [16] fp16.  Returns y [M, N]."""
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(wq, torch.int32, "wq")
    _need(absmax, torch.float16, "absmax")
    _need(lut, torch.float16, "lut")
    M, K = x.shape
    N = absmax.shape[0]
    need = packed_words(4, N, K)
    if need and wq.numel() != need:
        raise ValueError("wq does not hold N x K device-layout 4-bit codes")
    if lut.numel() != 16:
        raise ValueError("lut must hold 16 entries")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out")
    _check("qgemv_lut4", lib().qgemv_lut4(M, N, K, _ptr(x), _ptr(wq), _ptr(absmax), _ptr(lut), _ptr(out),
                                          _stream(x)))
    return out


def tilecoo_encode(N, K, rows, cols, vals):
    """Host-side Tile-COO encoding of fp16 outliers (numpy in, numpy out).

    rows, cols: integer coordinates; vals: fp16 values.  Returns (tile_ptr
    uint32 [ceil(N/16) * ceil(K/128) + 1]: tiles of 16 rows x 128 k, tile_rec
    uint32 [nnz])."""
    import numpy as np

    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    vbits = np.ascontiguousarray(np.asarray(vals, dtype=np.float16).view(np.uint16))
    nnz = rows.size
    if cols.size != nnz or vbits.size != nnz:
        raise ValueError("rows, cols and vals must have one entry per outlier")
    n_ptr = int(lib().qgemv_tilecoo_ptr_len(N, K))
    if n_ptr == 0:
        raise ValueError("bad N or K")
    ptr = np.zeros(n_ptr, dtype=np.uint32)
    rec = np.zeros(max(nnz, 1), dtype=np.uint32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check("qgemv_tilecoo_encode", lib().qgemv_tilecoo_encode(N, K, nnz, p(rows), p(cols), p(vbits), p(ptr), p(rec)))
    return ptr, rec[:nnz]


def outlier(x, wq, scales, zeros, tile_ptr, tile_rec, path=PATH_AUTO, out=None):
    """y = x . (W_dense + S)^T: the W4 uniform format plus fp16 Tile-COO outliers.

    tile_ptr / tile_rec: device int32 (or uint32 viewed as int32) tensors from
    tilecoo_encode.  Other arguments as uniform(..., bits=4)."""
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(wq, torch.int32, "wq")
    _need(scales, torch.float16, "scales")
    _need(zeros, torch.int32, "zeros")
    _need(tile_ptr, torch.int32, "tile_ptr")
    _need(tile_rec, torch.int32, "tile_rec")
    M, K = x.shape
    N = scales.shape[0]
    need = packed_words(4, N, K)
    if need and wq.numel() != need:
        raise ValueError("wq does not hold N x K device-layout 4-bit codes")
    if tile_ptr.numel() != int(lib().qgemv_tilecoo_ptr_len(N, K)):
        raise ValueError("tile_ptr does not match N x K")
    nnz = tile_rec.numel()
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out")
    rec_ptr = _ptr(tile_rec) if nnz else None
    _check("qgemv_outlier", lib().qgemv_outlier(path, M, N, K, _ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros),
                                                _ptr(tile_ptr), rec_ptr, nnz, _ptr(out), _stream(x)))
    return out


def codebook_workspace_bytes(M, N, K):
    return int(lib().qgemv_codebook_workspace_bytes(M, N, K))


def codebook(x, codes, cb, scales, ws=None, out=None):
    """y = x . dequant(codes)^T for a 256 x 4 fp16 codebook (8-bit codes, one
    per 4 consecutive k) with one fp16 scale per 128 k.

    codes: int32 words of the [N, K/4] uint8 code matrix packed with
    pack(codes, 8, LAYOUT_ROWS64); cb [256, 4] fp16; scales [N, K/128] fp16;
    ws: optional scratch workspace (a uint8/int32 tensor, contents not
    needed) of codebook_workspace_bytes(M, N, K) bytes, reusable across
    calls on one stream; with it K is split across workgroups."""
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(codes, torch.int32, "codes")
    _need(cb, torch.float16, "codebook")
    _need(scales, torch.float16, "scales")
    M, K = x.shape
    N = scales.shape[0]
    need = packed_words(8, N, K // 4, LAYOUT_ROWS64) if K % 512 == 0 else 0
    if need and codes.numel() != need:
        raise ValueError("codes do not hold the N x K/4 code matrix in the 64-row layout")
    if cb.numel() != 1024:
        raise ValueError("codebook must be 256 x 4")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out")
    ws_ptr, ws_bytes = (None, 0)
    if ws is not None:
        if not ws.is_cuda or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous CUDA tensor")
        ws_ptr, ws_bytes = _ptr(ws), ws.numel() * ws.element_size()
    _check("qgemv_codebook", lib().qgemv_codebook(M, N, K, _ptr(x), _ptr(codes), _ptr(cb), _ptr(scales), _ptr(out),
                                                  ws_ptr, ws_bytes, _stream(x)))
    return out


# ---------------------------------------------------------------------------
# unfused baselines (eager dequantization + dense GEMV; separate SpMV)
# ---------------------------------------------------------------------------

def _out_w(N, K, like, out):
    torch = _torch()
    if out is None:
        return torch.empty((N, K), dtype=torch.float16, device=like.device)
    _need(out, torch.float16, "out")
    if tuple(out.shape) != (N, K):
        raise ValueError("out must be [N, K]")
    return out


def dequant(wq, scales, zeros, bits, K, out=None):
    """Eager dequantization: fp16 W [N, K] row-major, w = s * (q - z), each
    weight the exact product rounded once.  Arguments as `uniform`."""
    torch = _torch()
    _need(wq, torch.int32, "wq")
    _need(scales, torch.float16, "scales")
    _need(zeros, torch.int32, "zeros")
    N = scales.shape[0]
    need = packed_words(bits, N, K)
    if need and wq.numel() != need:
        raise ValueError("wq does not hold N x K device-layout codes")
    out = _out_w(N, K, wq, out)
    _check("qgemv_dequant", lib().qgemv_dequant(bits, N, K, _ptr(wq), _ptr(scales), _ptr(zeros), _ptr(out),
                                                _stream(wq)))
    return out


def dequant_lut4(wq, absmax, lut, K, out=None):
    """Eager dequantization of 4-bit table codes: w = lut[q] * absmax[n, k/64]."""
    torch = _torch()
    _need(wq, torch.int32, "wq")
    _need(absmax, torch.float16, "absmax")
    _need(lut, torch.float16, "lut")
    N = absmax.shape[0]
    need = packed_words(4, N, K)
    if need and wq.numel() != need:
        raise ValueError("wq does not hold N x K device-layout 4-bit codes")
    if lut.numel() != 16:
        raise ValueError("lut must hold 16 entries")
    out = _out_w(N, K, wq, out)
    _check("qgemv_dequant_lut4", lib().qgemv_dequant_lut4(N, K, _ptr(wq), _ptr(absmax), _ptr(lut), _ptr(out),
                                                          _stream(wq)))
    return out


def gemv_f16(x, w, out=None):
    """Dense fp16 GEMV y = x . w^T (w [N, K] row-major), fp32 accumulation."""
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(w, torch.float16, "w")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("w must be [N, K]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out")
    _check("qgemv_gemv_f16", lib().qgemv_gemv_f16(M, N, K, _ptr(x), _ptr(w), _ptr(out), _stream(x)))
    return out


def spmv_tilecoo(x, tile_ptr, tile_rec, y):
    """y += x . S^T for Tile-COO outliers (in place on y [M, N]; returns y)."""
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(tile_ptr, torch.int32, "tile_ptr")
    _need(y, torch.float16, "y")
    M, K = x.shape
    N = y.shape[1]
    if tile_rec is not None:
        _need(tile_rec, torch.int32, "tile_rec")
    nnz = 0 if tile_rec is None else tile_rec.numel()
    if tile_ptr.numel() != int(lib().qgemv_tilecoo_ptr_len(N, K)):
        raise ValueError("tile_ptr does not match N x K")
    _check("qgemv_spmv_tilecoo", lib().qgemv_spmv_tilecoo(M, N, K, _ptr(x), _ptr(tile_ptr),
                                                          _ptr(tile_rec if nnz else None), nnz, _ptr(y),
                                                          _stream(x)))
    return y


# ---------------------------------------------------------------------------
# general codebook GEMV (m additive codebooks, vector length v, group g)
# ---------------------------------------------------------------------------

def pack_codebook_planes(codes):
    """[ncb, N, K/v] uint8 codes -> int32 words: the ncb planes, each packed in
    the 64-row layout, one after the other (the qgemv_codebook_gen format)."""
    torch = _torch()
    _need(codes, torch.uint8, "codes")
    return torch.cat([pack(codes[i].contiguous(), 8, LAYOUT_ROWS64) for i in range(codes.shape[0])])


def codebook_gen_workspace_bytes(M, N, K, ncb, v, group):
    return int(lib().qgemv_codebook_gen_workspace_bytes(M, N, K, ncb, v, group))


def codebook_gen(x, codes, codebooks, scales, group, ws=None, out=None):
    """y = x . W^T with w[n, v j + t] = scales[n, (v j + t)/group] * sum_i codebooks[i][codes_i[n, j]][t].

    codes: int32 words from pack_codebook_planes; codebooks [ncb, 256, v] fp16;
    scales [N, K/group] fp16; ws: optional device scratch of
    codebook_gen_workspace_bytes(...) bytes."""
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(codes, torch.int32, "codes")
    _need(codebooks, torch.float16, "codebooks")
    _need(scales, torch.float16, "scales")
    M, K = x.shape
    N = scales.shape[0]
    ncb, nc, v = codebooks.shape
    if nc != 256:
        raise ValueError("codebooks must be [ncb, 256, v]")
    need = packed_words(8, N, K // v, LAYOUT_ROWS64) * ncb if v and K % v == 0 else 0
    if need and codes.numel() != need:
        raise ValueError("codes do not hold ncb planes of N x K/v codes")
    if ws is not None and (not ws.is_cuda or not ws.is_contiguous()):
        raise ValueError("ws must be a contiguous CUDA tensor")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out")
    wsb = ws.numel() * ws.element_size() if ws is not None else 0
    _check("qgemv_codebook_gen", lib().qgemv_codebook_gen(M, N, K, ncb, v, group, _ptr(x), _ptr(codes),
                                                          _ptr(codebooks), _ptr(scales), _ptr(out), _ptr(ws),
                                                          wsb, _stream(x)))
    return out


def gemm_uniform(x, wq, scales, zeros, bits, out=None):
    """Prefill-size y = x . dequant(Wq)^T for any M (matrix cores); arguments
    as `uniform`, x [M, K] with M unbounded."""
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(wq, torch.int32, "wq")
    _need(scales, torch.float16, "scales")
    _need(zeros, torch.int32, "zeros")
    M, K = x.shape
    N = scales.shape[0]
    need = packed_words(bits, N, K)
    if need and wq.numel() != need:
        raise ValueError("wq does not hold N x K device-layout codes")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out")
    _check("qgemv_gemm_uniform", lib().qgemv_gemm_uniform(bits, M, N, K, _ptr(x), _ptr(wq), _ptr(scales),
                                                          _ptr(zeros), _ptr(out), _stream(x)))
    return out


def w4a8_workspace_bytes(M, K):
    return int(lib().qgemv_w4a8_workspace_bytes(M, K))


def w4a8_split_workspace_bytes(M, K):
    return int(lib().qgemv_w4a8_split_workspace_bytes(M, K))


def w4a8_asym_workspace_bytes(M, K):
    return int(lib().qgemv_w4a8_asym_workspace_bytes(M, K))


def w4a8_split(x, wq, scales, zeros, ws, out=None):
    """W4A8 by the split strategy (the int8 activations as two 4-bit slices
    on the fp8 matrix cores); the same bits as w4a8.  ws: at least
    w4a8_split_workspace_bytes(M, K) bytes."""
    return w4a8(x, wq, scales, zeros, ws, out, _fn="qgemv_w4a8_split")


def w4a8_asym(x, wq, scales, zeros, ws, out=None):
    """W4A8 with asymmetric int8 activations (a scale and a zero point per
    row), zero points of both operands by the expansion.  ws: at least
    w4a8_asym_workspace_bytes(M, K) bytes."""
    return w4a8(x, wq, scales, zeros, ws, out, _fn="qgemv_w4a8_asym")


def w4a8(x, wq, scales, zeros, ws, out=None, _fn="qgemv_w4a8"):
    """W4A8 with int8 activations (one symmetric scale per row) on the int8
    matrix cores.  Arguments as w4a16; ws: a CUDA tensor of at least
    w4a8_workspace_bytes(M, K) bytes (16-byte aligned), which holds the int8
    activations [M, K] and then the fp32 row scales after the call."""
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(wq, torch.int32, "wq")
    _need(scales, torch.float16, "scales")
    _need(zeros, torch.int32, "zeros")
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise TypeError("ws must be a contiguous CUDA tensor")
    M, K = x.shape
    N = scales.shape[0]
    need = packed_words(4, N, K)
    if need and wq.numel() != need:
        raise ValueError("wq does not hold N x K device-layout 4-bit codes")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out")
    _check(_fn, getattr(lib(), _fn)(M, N, K, _ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros), _ptr(out),
                                    _ptr(ws), ws.numel() * ws.element_size(), _stream(x)))
    return out


W4A8_NOALLOC_MAX_MK = 1 << 20  # QGEMV_W4A8_NOALLOC_MAX_MK


def w4a8_noalloc(x, wq, scales, zeros, out=None):
    """w4a8 without a workspace: the library's own per-GPU scratch holds the
    int8 activations (M * K <= W4A8_NOALLOC_MAX_MK).  Calls that overlap in
    time on one GPU race on that scratch."""
    torch = _torch()
    _need(x, torch.float16, "x")
    _need(wq, torch.int32, "wq")
    _need(scales, torch.float16, "scales")
    _need(zeros, torch.int32, "zeros")
    M, K = x.shape
    N = scales.shape[0]
    need = packed_words(4, N, K)
    if need and wq.numel() != need:
        raise ValueError("wq does not hold N x K device-layout 4-bit codes")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float16, device=x.device)
    else:
        _need(out, torch.float16, "out")
    _check("qgemv_w4a8_noalloc", lib().qgemv_w4a8_noalloc(M, N, K, _ptr(x), _ptr(wq), _ptr(scales), _ptr(zeros),
                                                          _ptr(out), _stream(x)))
    return out


def stream_read(buf, sink, nbytes=None, workgroups=1024, threads=512, offset=0):
    """Measurement: read `nbytes` of the CUDA tensor `buf` from byte `offset`
    once (qgemv_stream_read); sink: a CUDA tensor of at least 4 bytes."""
    torch = _torch()
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous CUDA tensor")
    total = buf.numel() * buf.element_size()
    nbytes = total - offset if nbytes is None else nbytes
    if offset < 0 or offset + nbytes > total:
        raise ValueError("range outside buf")
    _check("qgemv_stream_read", lib().qgemv_stream_read(_vp(buf.data_ptr() + offset), nbytes, _ptr(sink),
                                                        workgroups, threads, _stream(buf)))
