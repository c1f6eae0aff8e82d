"""The C-ABI library loads on a CPU-only host, exports every symbol the header
declares, and its host-side logic (validation, status strings, sizes) works
without touching a GPU."""
import ctypes
import os
import re

import pytest

import gemm_unpack_bit_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(qgemv_\w+)\s*\(", src))
    return names


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(q.LIB_PATH):
        pytest.skip("library not built")
    return q.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 10
    raw = ctypes.CDLL(q.LIB_PATH)
    for n in sorted(names):
        assert hasattr(raw, n), n
    # and the binding's signature table covers exactly the header
    assert set(q._SIGS) == names


def test_host_queries(L):
    assert L.qgemv_version() >= 100
    for s in range(8):
        assert L.qgemv_status_string(s)
    assert L.qgemv_status_string(99) == b"unknown status"
    assert L.qgemv_packed_words(4, 0, 3, 4096) == 3 * 512
    assert L.qgemv_packed_words(2, 0, 5, 17) == 5 * 2
    assert L.qgemv_packed_words(8, 0, 2, 3) == 2
    assert L.qgemv_packed_words(3, 0, 2, 3) == 0
    assert L.qgemv_packed_words(4, 1, 20, 256) == 32 * 256 * 4 // 32   # rows padded to 16
    assert L.qgemv_packed_words(2, 1, 16, 128) == 16 * 128 * 2 // 32
    assert L.qgemv_packed_words(4, 1, 20, 100) == 0                   # cols % 128
    assert L.qgemv_packed_words(4, 2, 20, 256) == 0                   # unknown layout
    assert L.qgemv_last_hip_error() == 0


def test_layout_version_and_workspace_query(L):
    assert L.qgemv_layout_version() == q.LAYOUT_VERSION == 1
    hdr = open(os.path.join(ROOT, "include", "qgemv.h")).read()
    assert re.search(r"#define QGEMV_LAYOUT_VERSION 1\b", hdr)
    # formats that take no workspace
    for v in (q.W2, q.W4, q.W8, q.LUT4, q.OUTLIER4):
        assert L.qgemv_workspace_bytes(v, 1, 4096, 4096) == 0
        assert L.qgemv_workspace_bytes(v, 16, 57344, 8192) == 0
    # the families with one agree with their own queries
    for M, N, K in ((1, 4096, 4096), (4, 57344, 8192), (16, 8192, 28672)):
        assert L.qgemv_workspace_bytes(q.CODEBOOK, M, N, K) == L.qgemv_codebook_workspace_bytes(M, N, K)
        assert L.qgemv_workspace_bytes(q.W4A8, M, N, K) == L.qgemv_w4a8_workspace_bytes(M, K) > 0
    # unknown variant, bad shapes
    assert L.qgemv_workspace_bytes(3, 1, 64, 128) == 0
    assert L.qgemv_workspace_bytes(q.W4A8, 0, 64, 128) == 0
    assert L.qgemv_workspace_bytes(q.W4A8, 1, 64, 100) == 0
    assert L.qgemv_workspace_bytes(q.W4A8, 1, 0, 128) == 0


FAKE = 0x1000  # 16-byte aligned, never dereferenced: every call below fails validation first


def _uni(L, bits=4, path=0, M=1, N=64, K=256, x=FAKE, wq=FAKE * 2, s=FAKE * 3, z=FAKE * 4, y=FAKE * 64):
    v = ctypes.c_void_p
    return L.qgemv_uniform(bits, path, M, N, K, v(x), v(wq), v(s), v(z), v(y), v(0))


def test_uniform_validation_without_gpu(L):
    assert _uni(L, x=0) == q.ERR_NULL
    assert _uni(L, y=0) == q.ERR_NULL
    assert _uni(L, bits=3) == q.ERR_UNSUPPORTED
    assert _uni(L, path=7) == q.ERR_UNSUPPORTED
    assert _uni(L, M=0) == q.ERR_SHAPE
    assert _uni(L, M=17) == q.ERR_SHAPE
    assert _uni(L, N=0) == q.ERR_SHAPE
    assert _uni(L, K=200) == q.ERR_SHAPE
    assert _uni(L, K=0) == q.ERR_SHAPE
    assert _uni(L, x=FAKE + 2) == q.ERR_ALIGN
    assert _uni(L, wq=FAKE * 2 + 8) == q.ERR_ALIGN
    assert _uni(L, y=FAKE * 2) == q.ERR_VALUE  # y overlaps wq
    v = ctypes.c_void_p
    assert L.qgemv_w4a16(1, 64, 256, v(0), v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(0)) == q.ERR_NULL
    assert L.qgemv_w2a16(0, 64, 256, v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(0)) == q.ERR_SHAPE
    assert L.qgemv_w8a16(1, 64, 100, v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(FAKE), v(0)) == q.ERR_SHAPE


def test_pack_validation_without_gpu(L):
    v = ctypes.c_void_p
    assert L.qgemv_pack(4, 1, 2, 128, v(0), v(FAKE), v(0)) == q.ERR_NULL
    assert L.qgemv_pack(5, 1, 2, 128, v(FAKE), v(FAKE * 16), v(0)) == q.ERR_UNSUPPORTED
    assert L.qgemv_pack(4, 2, 2, 128, v(FAKE), v(FAKE * 16), v(0)) == q.ERR_UNSUPPORTED  # layout
    assert L.qgemv_pack(4, 0, -1, 8, v(FAKE), v(FAKE * 16), v(0)) == q.ERR_SHAPE
    assert L.qgemv_pack(4, 1, 2, 8, v(FAKE), v(FAKE * 16), v(0)) == q.ERR_SHAPE       # device needs cols % 128
    assert L.qgemv_unpack(4, 1, 2, 128, v(FAKE), v(0), v(0)) == q.ERR_NULL
    assert L.qgemv_pack(4, 0, 2, 8, v(FAKE), v(FAKE + 4), v(0)) == q.ERR_VALUE  # overlap


def _lut(L, M=1, N=64, K=256, x=FAKE, wq=FAKE * 2, a=FAKE * 3, lut=FAKE * 4, y=FAKE * 64):
    v = ctypes.c_void_p
    return L.qgemv_lut4(M, N, K, v(x), v(wq), v(a), v(lut), v(y), v(0))


def test_lut4_validation_without_gpu(L):
    assert _lut(L, lut=0) == q.ERR_NULL
    assert _lut(L, a=0) == q.ERR_NULL
    assert _lut(L, M=17) == q.ERR_SHAPE
    assert _lut(L, K=192) == q.ERR_SHAPE        # the tiles are 128 wide
    assert _lut(L, K=48128) == q.ERR_SHAPE      # beyond the on-chip activation staging
    assert _lut(L, x=FAKE + 4) == q.ERR_ALIGN
    assert _lut(L, a=FAKE * 3 + 1) == q.ERR_ALIGN
    assert _lut(L, y=FAKE * 4) == q.ERR_VALUE    # y overlaps the table


def _cb(L, M=1, N=64, K=512, x=FAKE, codes=FAKE * 2, cbk=FAKE * 3, s=FAKE * 4, y=FAKE * 64, ws=0, wsb=0):
    v = ctypes.c_void_p
    return L.qgemv_codebook(M, N, K, v(x), v(codes), v(cbk), v(s), v(y), v(ws), wsb, v(0))


def test_codebook_validation_without_gpu(L):
    assert _cb(L, codes=0) == q.ERR_NULL
    assert _cb(L, K=384) == q.ERR_SHAPE          # K must be a multiple of 512
    assert _cb(L, M=0) == q.ERR_SHAPE
    assert _cb(L, x=FAKE + 8) == q.ERR_ALIGN
    assert _cb(L, cbk=FAKE * 3 + 2) == q.ERR_ALIGN
    assert _cb(L, y=FAKE * 3) == q.ERR_VALUE      # y overlaps the codebook
    assert _cb(L, ws=FAKE * 4, wsb=64) == q.ERR_VALUE  # the workspace overlaps the scales
    assert L.qgemv_codebook_workspace_bytes(1, 64, 384) == 0
    n = L.qgemv_codebook_workspace_bytes(1, 8192, 28672)
    assert n >= 2 * 4 * 8192                       # few rows, long K: split, one fp32 partial per row and split


def test_unfused_validation_without_gpu(L):
    v = ctypes.c_void_p
    dq = lambda bits=4, N=64, K=256, wq=FAKE, s=FAKE * 2, z=FAKE * 3, w=FAKE * 64: L.qgemv_dequant(
        bits, N, K, v(wq), v(s), v(z), v(w), v(0))
    assert dq(wq=0) == q.ERR_NULL
    assert dq(bits=3) == q.ERR_UNSUPPORTED
    assert dq(K=200) == q.ERR_SHAPE
    assert dq(N=0) == q.ERR_SHAPE
    assert dq(N=1 << 20, K=1 << 10) == q.ERR_SHAPE      # fp16 W of 2 GiB
    assert dq(w=FAKE * 64 + 8) == q.ERR_ALIGN
    assert dq(s=FAKE * 2 + 1) == q.ERR_ALIGN
    assert dq(w=FAKE * 2) == q.ERR_VALUE                 # W overlaps the scales
    dl = lambda N=64, K=256, wq=FAKE, a=FAKE * 2, lut=FAKE * 3, w=FAKE * 64: L.qgemv_dequant_lut4(
        N, K, v(wq), v(a), v(lut), v(w), v(0))
    assert dl(lut=0) == q.ERR_NULL
    assert dl(K=64) == q.ERR_SHAPE
    assert dl(wq=FAKE + 4) == q.ERR_ALIGN
    assert dl(w=FAKE * 3) == q.ERR_VALUE                 # W overlaps the table
    gf = lambda M=1, N=64, K=256, x=FAKE, w=FAKE * 2, y=FAKE * 1024: L.qgemv_gemv_f16(
        M, N, K, v(x), v(w), v(y), v(0))
    assert gf(w=0) == q.ERR_NULL
    assert gf(M=17) == q.ERR_SHAPE
    assert gf(K=100) == q.ERR_SHAPE
    assert gf(x=FAKE + 2) == q.ERR_ALIGN
    assert gf(y=FAKE * 2 + 32) == q.ERR_VALUE            # y inside W
    sp = lambda M=1, N=64, K=256, x=FAKE, p=FAKE * 2, r=FAKE * 3, nnz=10, y=FAKE * 64: L.qgemv_spmv_tilecoo(
        M, N, K, v(x), v(p), v(r), nnz, v(y), v(0))
    assert sp(r=0) == q.ERR_NULL
    assert sp(K=2 * 1048576) == q.ERR_SHAPE              # beyond the on-chip tile_ptr staging
    assert sp(nnz=-1) == q.ERR_SHAPE
    assert sp(nnz=64 * 256 + 1) == q.ERR_SHAPE
    assert sp(p=FAKE * 2 + 2) == q.ERR_ALIGN
    assert sp(y=FAKE * 3) == q.ERR_VALUE                 # y overlaps the records
    assert sp(r=0, nnz=0) == q.OK                        # nothing to add: no launch


def test_codebook_gen_validation_without_gpu(L):
    v_ = ctypes.c_void_p

    def cg(M=1, N=64, K=512, ncb=1, v=4, g=128, x=FAKE, codes=FAKE * 2, cbk=FAKE * 3, s=FAKE * 4, y=FAKE * 64,
           ws=0, wsb=0):
        return L.qgemv_codebook_gen(M, N, K, ncb, v, g, v_(x), v_(codes), v_(cbk), v_(s), v_(y), v_(ws), wsb, v_(0))

    assert cg(codes=0) == q.ERR_NULL
    assert cg(v=6) == q.ERR_UNSUPPORTED
    assert cg(ncb=2, v=4) == q.ERR_UNSUPPORTED      # more than 2 code bits per weight
    assert cg(g=16) == q.ERR_UNSUPPORTED
    assert cg(K=384) == q.ERR_SHAPE                 # K must be a multiple of 256
    assert cg(M=17) == q.ERR_SHAPE
    assert cg(x=FAKE + 4) == q.ERR_ALIGN
    assert cg(codes=FAKE * 2 + 8) == q.ERR_ALIGN
    assert cg(y=FAKE * 3) == q.ERR_VALUE            # y overlaps the codebooks
    assert cg(ws=FAKE * 4, wsb=64) == q.ERR_VALUE   # the workspace overlaps the scales
    assert L.qgemv_codebook_gen_workspace_bytes(1, 64, 512, 2, 4, 128) == 0
    assert L.qgemv_codebook_gen_workspace_bytes(1, 4096, 4096, 3, 16, 32) >= 4 * 4096


def test_gemm_validation_without_gpu(L):
    v = ctypes.c_void_p
    gm = lambda bits=4, M=100, N=64, K=256, x=FAKE, wq=FAKE * 2, s=FAKE * 3, z=FAKE * 4, y=FAKE * 1024: \
        L.qgemv_gemm_uniform(bits, M, N, K, v(x), v(wq), v(s), v(z), v(y), v(0))
    assert gm(wq=0) == q.ERR_NULL
    assert gm(bits=3) == q.ERR_UNSUPPORTED
    assert gm(M=0) == q.ERR_SHAPE
    assert gm(K=200) == q.ERR_SHAPE
    assert gm(x=FAKE + 8) == q.ERR_ALIGN
    assert gm(y=FAKE * 3) == q.ERR_VALUE             # y overlaps the scales


def test_w4a8_validation_without_gpu(L):
    v = ctypes.c_void_p
    wa = lambda M=1, N=64, K=256, x=FAKE, wq=FAKE * 2, s=FAKE * 3, z=FAKE * 4, y=FAKE * 64, ws=FAKE * 128, wsb=1 << 16: \
        L.qgemv_w4a8(M, N, K, v(x), v(wq), v(s), v(z), v(y), v(ws), wsb, v(0))
    assert wa(x=0) == q.ERR_NULL
    assert wa(M=17) == q.ERR_SHAPE
    assert wa(ws=0) == q.ERR_WORKSPACE
    assert wa(wsb=16) == q.ERR_WORKSPACE
    assert wa(ws=FAKE * 128 + 4) == q.ERR_ALIGN
    assert wa(x=FAKE + 8) == q.ERR_ALIGN
    assert wa(ws=FAKE * 2) == q.ERR_VALUE            # the workspace overlaps the codes
    assert L.qgemv_w4a8_workspace_bytes(3, 256) == 3 * 256 + 3 * 4   # int8 rows, then the fp32 scales


def test_w4a8_noalloc_validation_without_gpu(L):
    """Every check runs before the library looks up its scratch on the device."""
    v = ctypes.c_void_p
    na = lambda M=1, N=64, K=256, x=FAKE, wq=FAKE * 2, s=FAKE * 3, z=FAKE * 4, y=FAKE * 64: \
        L.qgemv_w4a8_noalloc(M, N, K, v(x), v(wq), v(s), v(z), v(y), v(0))
    assert na(x=0) == q.ERR_NULL
    assert na(M=17) == q.ERR_SHAPE
    assert na(K=200) == q.ERR_SHAPE
    # M * K beyond the scratch the library holds
    assert na(M=16, K=q.W4A8_NOALLOC_MAX_MK // 16 + 128, y=FAKE * 4096) == q.ERR_WORKSPACE
    assert na(M=1, K=q.W4A8_NOALLOC_MAX_MK + 128, y=FAKE * 4096) == q.ERR_WORKSPACE


def test_w4a8_split_and_asym_validation_without_gpu(L):
    v = ctypes.c_void_p
    for fn, wsq in ((L.qgemv_w4a8_split, L.qgemv_w4a8_split_workspace_bytes),
                    (L.qgemv_w4a8_asym, L.qgemv_w4a8_asym_workspace_bytes)):
        call = lambda M=1, N=64, K=256, x=FAKE, ws=FAKE * 128, wsb=1 << 16: \
            fn(M, N, K, v(x), v(FAKE * 2), v(FAKE * 3), v(FAKE * 4), v(FAKE * 64), v(ws), wsb, v(0))
        assert call(x=0) == q.ERR_NULL
        assert call(M=17) == q.ERR_SHAPE
        assert call(ws=0) == q.ERR_WORKSPACE
        assert call(wsb=wsq(1, 256) - 1) == q.ERR_WORKSPACE
        assert call(ws=FAKE * 2) == q.ERR_VALUE
    # split: two byte planes then the scales; asym: bytes, 16 scales, 16 zero points, [K/128][16] sums
    assert L.qgemv_w4a8_split_workspace_bytes(3, 256) == 2 * 768 + 12
    assert L.qgemv_w4a8_asym_workspace_bytes(3, 256) == 768 + 64 + 64 + 2 * 64
    assert L.qgemv_workspace_bytes(q.W4A8_SPLIT, 3, 64, 256) == L.qgemv_w4a8_split_workspace_bytes(3, 256)
    assert L.qgemv_workspace_bytes(q.W4A8_ASYM, 3, 64, 256) == L.qgemv_w4a8_asym_workspace_bytes(3, 256)
