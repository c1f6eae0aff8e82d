// C ABI of libqgemv.so: argument validation, dispatch and launch.
// Host-only code (built with the host compiler); kernels live in the .hip files.
#include "qgemv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kernels.hpp"

namespace qg {
const char* tune_env(const char* name) {
  static const bool on = std::getenv("QGEMV_TUNING") != nullptr;
  return on ? std::getenv(name) : nullptr;
}
}  // namespace qg

namespace {

thread_local int g_last_hip_error = 0;

// qgemv_gemm_uniform: batches of at most this many rows run as 16-row slices
// of the decode kernel
constexpr int QGEMV_GEMM_SLICE_MAX_M = 64;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return QGEMV_OK;
  g_last_hip_error = (int)e;
  return QGEMV_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool valid_bits(int b) { return b == 2 || b == 4 || b == 8; }

size_t words(int bits, int layout, int rows, int cols) { return qg::packed_words(bits, layout, rows, cols); }

// Shape rules shared by the compute entry points.  Kernels address every
// buffer with 32-bit byte offsets below 2^31 (buffer loads past the end read
// zero), so each operand must stay under 2 GiB.
int check_mnk(int M, int N, int K, int bits) {
  if (M < 1 || M > QGEMV_MAX_M || N < 1 || K < QGEMV_GROUP || K % QGEMV_GROUP) return QGEMV_ERR_SHAPE;
  const long lim = 1L << 31;
  if ((long)((N + 15) / 16) * 16 * K * bits / 8 >= lim || (long)M * K * 2 >= lim || (long)M * N * 2 >= lim)
    return QGEMV_ERR_SHAPE;
  return QGEMV_OK;
}

// Tuning overrides (QGEMV_*_CFG and the like) are looked up only when
// QGEMV_TUNING was set at the first call of the process, so normal calls do no
// environment lookups on the host path; when it is set they are read on every
// call, so a sweep can change them between calls.
using qg::tune_env;

// The out-of-range flag of qgemv_pack is one device word: clearing it,
// packing and reading it back are serialized across host threads.
std::mutex g_pack_mutex;

// Tuning override of the launch shape: QGEMV_TILE_CFG="tpw,wk[,mt[,v]]"
// (tile-rows per workgroup, waves per workgroup, batch rows per VALU
// workgroup, pipeline variant).
qg::TileCfg tile_cfg(int bits, int M, int N, int K, bool mfma) {
  qg::TileCfg c = qg::pick_tiles(bits, M, N, K, mfma);
  if (const char* e = tune_env("QGEMV_TILE_CFG")) {
    int tpw, wk, mt, v;
    const int n = std::sscanf(e, "%d,%d,%d,%d", &tpw, &wk, &mt, &v);
    if (n >= 2) {
      c.tpw = tpw;
      c.wk = wk;
    }
    if (n >= 3 && !mfma) c.mt = mt;
    if (n >= 4) c.v = v;
  }
  return c;
}

// Workgroups of the prefill GEMM with 16 mi-row x 64 nt-column blocks.
long gemm_wgs(int M, int N, int mi, int nt) {
  return (long)((M + 16 * mi - 1) / (16 * mi)) * (((N + 15) / 16 + 4 * nt - 1) / (4 * nt));
}

// Prefill GEMM block (sweeps of the 8B and 70B layers, M = 32..2048, W2 /
// W4 / W8): the largest block that still gives enough workgroups, and on a
// thin grid two K halves per workgroup (twice the waves, same workgroups).
// 64 x 256 needs at least 400 workgroups (a narrower grid leaves one wave
// per SIMD with its loads, dequantization and MFMAs in series), 64 x 128 at
// least 384 with all of K, or 144 to 256 with two K halves (their 8-wave
// workgroups run one per CU, so more than 256 leave a tail: 70B q at M = 256
// 81.6 vs 71.2 us), else 32 x 128 (two K halves below 512).  64-row blocks only where they pad M by at most a quarter more
// than 32-row blocks.  8-bit weights have 32-row blocks only: 32 x 256 from
// 448 workgroups, else 32 x 128, with two K halves below 640.  (Two K
// halves need K/128 even; the caller falls back to one.)
void gemm_block(int bits, int M, int N, int& mi, int& nt, int& kh) {
  const bool m64 = (M + 63) / 64 * 64 * 4 <= (M + 31) / 32 * 32 * 5;
  kh = 1;
  if (bits == 8) {
    mi = 2;
    nt = gemm_wgs(M, N, 2, 4) >= 448 ? 4 : 2;
    if (nt == 2 && gemm_wgs(M, N, 2, 2) < 640) kh = 2;
  } else if (m64 && gemm_wgs(M, N, 4, 4) >= 400) {
    mi = 4, nt = 4;
  } else if (m64 && gemm_wgs(M, N, 4, 2) >= 384) {
    mi = 4, nt = 2;
  } else if (m64 && gemm_wgs(M, N, 4, 2) >= 144 && gemm_wgs(M, N, 4, 2) <= 256) {
    mi = 4, nt = 2, kh = 2;  // (8-wave workgroups run one per CU: at most one round)
  } else {
    mi = 2, nt = 2;
    kh = gemm_wgs(M, N, 2, 2) < 512 ? 2 : 1;
  }
}

// 17..64 rows: the 16-row slices of the decode kernel or the GEMM.  A slice
// streams the weights once, in about max(0.15 G + 2, weight bytes / 3.5
// TB/s) us (its per-workgroup group loop, or HBM; 2-bit codes priced as
// 4-bit ones: their unpack, not their bytes, bounds them); the GEMM's few
// workgroups (two K halves each) run the K loop, about 0.44 G us per 320
// workgroups.  Fitted to the 8B and 70B layers at M = 24..64 (W2 / W4 /
// W8): the GEMM takes the wide gate+up layers from M = 17 and the others
// from M = 48.
bool prefer_slices(int bits, int M, int N, int K) {
  if (M <= QGEMV_MAX_M) return true;
  if (M > QGEMV_GEMM_SLICE_MAX_M) return false;
  const int G = K / QGEMV_GROUP;
  const double wbytes = (double)N * K * (bits < 4 ? 4 : bits) / 8;
  const double t16 = std::max(0.15 * G + 2.0, wbytes / 3.5e6);
  int mi, nt, kh;
  gemm_block(bits, M, N, mi, nt, kh);
  const double rounds = std::max(1.0, (double)gemm_wgs(M, N, mi, nt) / 320.0);
  return (double)((M + QGEMV_MAX_M - 1) / QGEMV_MAX_M) * t16 <= 0.44 * G * rounds;
}

// Tuning override of the LUT4 launch shape: QGEMV_LUT4_CFG="tpw,ng,wk[,mt[,d]]".
qg::Lut4Cfg lut4_cfg(int M, int N, int K) {
  qg::Lut4Cfg c = qg::pick_lut4(M, N, K);
  if (const char* e = tune_env("QGEMV_LUT4_CFG")) {
    int tpw, ng, wk, mt, d;
    const int n = std::sscanf(e, "%d,%d,%d,%d,%d", &tpw, &ng, &wk, &mt, &d);
    if (n >= 3) {
      c.tpw = tpw;
      c.ng = ng;
      c.wk = wk;
    }
    if (n >= 4) c.mt = mt;
    if (n >= 5) c.d = d;
  }
  return c;
}

// Dot engine for QGEMV_PATH_AUTO, from the same sweeps: the VALU engine for
// one activation row; the MFMA engine from two rows on, where one matrix-core
// pass serves all rows (with activations staged in LDS it beats the two-row
// VALU engine on every measured layer, e.g. 70B down 27.4 vs 37.9 us).
int auto_path(int bits, int M, int N) {
  (void)bits;
  (void)N;
  return M <= 1 ? QGEMV_PATH_VALU : QGEMV_PATH_MFMA;
}

}  // namespace

extern "C" {

int qgemv_version(void) { return 200; }

int qgemv_layout_version(void) { return QGEMV_LAYOUT_VERSION; }

size_t qgemv_workspace_bytes(int variant, int M, int N, int K) {
  switch (variant) {
    case QGEMV_W2:
    case QGEMV_W4:
    case QGEMV_W8:
    case QGEMV_LUT4:
    case QGEMV_OUTLIER4: return 0;
    case QGEMV_CODEBOOK: return qgemv_codebook_workspace_bytes(M, N, K);
    case QGEMV_W4A8: return N >= 1 ? qgemv_w4a8_workspace_bytes(M, K) : 0;
    case QGEMV_W4A8_SPLIT: return N >= 1 ? qgemv_w4a8_split_workspace_bytes(M, K) : 0;
    case QGEMV_W4A8_ASYM: return N >= 1 ? qgemv_w4a8_asym_workspace_bytes(M, K) : 0;
  }
  return 0;
}

const char* qgemv_status_string(int status) {
  switch (status) {
    case QGEMV_OK: return "ok";
    case QGEMV_ERR_NULL: return "null pointer";
    case QGEMV_ERR_SHAPE: return "unsupported shape";
    case QGEMV_ERR_ALIGN: return "misaligned pointer";
    case QGEMV_ERR_UNSUPPORTED: return "unsupported variant or path";
    case QGEMV_ERR_WORKSPACE: return "workspace missing or too small";
    case QGEMV_ERR_VALUE: return "invalid data or aliasing output";
    case QGEMV_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int qgemv_last_hip_error(void) { return g_last_hip_error; }

size_t qgemv_packed_words(int bits, int layout, int rows, int cols) {
  if (!valid_bits(bits) || rows < 0 || cols < 0) return 0;
  if (layout == QGEMV_LAYOUT_DEVICE && cols % QGEMV_GROUP) return 0;
  if (layout != QGEMV_LAYOUT_PLAIN && layout != QGEMV_LAYOUT_DEVICE && layout != QGEMV_LAYOUT_ROWS64) return 0;
  return words(bits, layout, rows, cols);
}

int qgemv_pack(int bits, int layout, int rows, int cols, const uint8_t* codes, uint32_t* packed,
               qgemv_stream_t stream) {
  if (!codes || !packed) return QGEMV_ERR_NULL;
  if (!valid_bits(bits) || (layout != QGEMV_LAYOUT_PLAIN && layout != QGEMV_LAYOUT_DEVICE &&
                            !(layout == QGEMV_LAYOUT_ROWS64 && bits == 8)))
    return QGEMV_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || (layout == QGEMV_LAYOUT_DEVICE && cols % QGEMV_GROUP)) return QGEMV_ERR_SHAPE;
  if (overlaps(codes, (size_t)rows * cols, packed, words(bits, layout, rows, cols) * 4)) return QGEMV_ERR_VALUE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  std::lock_guard<std::mutex> lock(g_pack_mutex);
  int rc = hip_status(qg::launch_pack(bits, layout, rows, cols, codes, packed, s));
  if (rc) return rc;
  int bad = 0;
  rc = hip_status(qg::pack_error_flag(&bad, s));
  if (rc) return rc;
  return bad ? QGEMV_ERR_VALUE : QGEMV_OK;
}

int qgemv_unpack(int bits, int layout, int rows, int cols, const uint32_t* packed, uint8_t* codes,
                 qgemv_stream_t stream) {
  if (!codes || !packed) return QGEMV_ERR_NULL;
  if (!valid_bits(bits) || (layout != QGEMV_LAYOUT_PLAIN && layout != QGEMV_LAYOUT_DEVICE &&
                            !(layout == QGEMV_LAYOUT_ROWS64 && bits == 8)))
    return QGEMV_ERR_UNSUPPORTED;
  if (rows < 0 || cols < 0 || (layout == QGEMV_LAYOUT_DEVICE && cols % QGEMV_GROUP)) return QGEMV_ERR_SHAPE;
  if (overlaps(codes, (size_t)rows * cols, packed, words(bits, layout, rows, cols) * 4)) return QGEMV_ERR_VALUE;
  return hip_status(
      qg::launch_unpack(bits, layout, rows, cols, packed, codes, reinterpret_cast<hipStream_t>(stream)));
}

int qgemv_uniform(int bits, int path, int M, int N, int K, const uint16_t* x, const uint32_t* wq,
                  const uint16_t* scales, const uint32_t* zeros, uint16_t* y, qgemv_stream_t stream) {
  if (!x || !wq || !scales || !zeros || !y) return QGEMV_ERR_NULL;
  if (!valid_bits(bits)) return QGEMV_ERR_UNSUPPORTED;
  if (path != QGEMV_PATH_AUTO && path != QGEMV_PATH_VALU && path != QGEMV_PATH_MFMA)
    return QGEMV_ERR_UNSUPPORTED;
  int rc = check_mnk(M, N, K, bits);
  if (rc) return rc;
  if (!aligned16(x) || !aligned16(wq) || ((uintptr_t)scales & 1u) || ((uintptr_t)zeros & 3u) ||
      ((uintptr_t)y & 1u))
    return QGEMV_ERR_ALIGN;
  const size_t ybytes = (size_t)M * N * 2;
  const int G = K / QGEMV_GROUP;
  if (overlaps(y, ybytes, x, (size_t)M * K * 2) ||
      overlaps(y, ybytes, wq, words(bits, QGEMV_LAYOUT_DEVICE, N, K) * 4) ||
      overlaps(y, ybytes, scales, (size_t)N * G * 2) ||
      overlaps(y, ybytes, zeros, words(bits, QGEMV_LAYOUT_PLAIN, N, G) * 4))
    return QGEMV_ERR_VALUE;
  qg::UniformArgs a{bits, M, N, K, x, wq, scales, zeros, y};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (path == QGEMV_PATH_AUTO) path = auto_path(bits, M, N);
  const bool mfma = path == QGEMV_PATH_MFMA;
  return hip_status(qg::launch_gemv_tiles(a, tile_cfg(bits, M, N, K, mfma), s));
}

size_t qgemv_w4a8_workspace_bytes(int M, int K) {
  if (M < 1 || M > QGEMV_MAX_M || K < QGEMV_GROUP || K % QGEMV_GROUP) return 0;
  return qg::w4a8_ws_bytes(M, K);
}

namespace {
// qgemv_w4a8 (and its split / asymmetric forms) and qgemv_w4a8_noalloc:
// argument checks (null, shape, workspace, alignment, overlap), then the two
// kernels with `ws` as the scratch.  `ws_checked` = false skips the
// workspace overlap test (library scratch).
int w4a8_call(int M, int N, int K, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
              const uint32_t* zeros, uint16_t* y, void* ws, size_t ws_bytes, bool ws_checked,
              qgemv_stream_t stream, int mode = qg::W4A8_PAD) {
  const qg::W4A8Ws lay = qg::w4a8_ws_layout(mode, M, K);
  if (!ws || ws_bytes < lay.total) return QGEMV_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(wq) || ((uintptr_t)scales & 1u) || ((uintptr_t)zeros & 3u) ||
      ((uintptr_t)y & 1u) || !aligned16(ws))
    return QGEMV_ERR_ALIGN;
  const size_t ybytes = (size_t)M * N * 2, G = K / QGEMV_GROUP;
  const size_t in_b[4] = {(size_t)M * K * 2, words(4, QGEMV_LAYOUT_DEVICE, N, K) * 4, G * N * 2,
                          words(4, QGEMV_LAYOUT_PLAIN, N, (int)G) * 4};
  const void* in_p[4] = {x, wq, scales, zeros};
  for (int i = 0; i < 4; ++i)
    if (overlaps(y, ybytes, in_p[i], in_b[i]) || (ws_checked && overlaps(ws, ws_bytes, in_p[i], in_b[i])))
      return QGEMV_ERR_VALUE;
  if (ws_checked && overlaps(ws, ws_bytes, y, ybytes)) return QGEMV_ERR_VALUE;
  char* w = reinterpret_cast<char*>(ws);
  qg::W4A8Args a{M, N, K, x, wq, scales, zeros, y, reinterpret_cast<int8_t*>(w + lay.xq),
                 reinterpret_cast<float*>(w + lay.sx), mode,
                 mode == qg::W4A8_SPLIT ? reinterpret_cast<uint8_t*>(w + lay.xl) : nullptr,
                 mode == qg::W4A8_ASYM ? reinterpret_cast<int*>(w + lay.zx) : nullptr,
                 mode == qg::W4A8_ASYM ? reinterpret_cast<int*>(w + lay.xsum) : nullptr};
  int wk = qg::w4a8_waves(N, K);
  if (const char* e = tune_env("QGEMV_W4A8_WK")) wk = std::atoi(e);  // tuning override
  return hip_status(qg::launch_gemv_w4a8(a, wk, reinterpret_cast<hipStream_t>(stream)));
}
}  // namespace

int qgemv_w4a8(int M, int N, int K, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
               const uint32_t* zeros, uint16_t* y, void* ws, size_t ws_bytes, qgemv_stream_t stream) {
  if (!x || !wq || !scales || !zeros || !y) return QGEMV_ERR_NULL;
  int rc = check_mnk(M, N, K, 4);
  if (rc) return rc;
  return w4a8_call(M, N, K, x, wq, scales, zeros, y, ws, ws_bytes, true, stream);
}

size_t qgemv_w4a8_split_workspace_bytes(int M, int K) {
  if (M < 1 || M > QGEMV_MAX_M || K < QGEMV_GROUP || K % QGEMV_GROUP) return 0;
  return qg::w4a8_ws_layout(qg::W4A8_SPLIT, M, K).total;
}

int qgemv_w4a8_split(int M, int N, int K, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                     const uint32_t* zeros, uint16_t* y, void* ws, size_t ws_bytes, qgemv_stream_t stream) {
  if (!x || !wq || !scales || !zeros || !y) return QGEMV_ERR_NULL;
  int rc = check_mnk(M, N, K, 4);
  if (rc) return rc;
  return w4a8_call(M, N, K, x, wq, scales, zeros, y, ws, ws_bytes, true, stream, qg::W4A8_SPLIT);
}

size_t qgemv_w4a8_asym_workspace_bytes(int M, int K) {
  if (M < 1 || M > QGEMV_MAX_M || K < QGEMV_GROUP || K % QGEMV_GROUP) return 0;
  return qg::w4a8_ws_layout(qg::W4A8_ASYM, M, K).total;
}

int qgemv_w4a8_asym(int M, int N, int K, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                    const uint32_t* zeros, uint16_t* y, void* ws, size_t ws_bytes, qgemv_stream_t stream) {
  if (!x || !wq || !scales || !zeros || !y) return QGEMV_ERR_NULL;
  int rc = check_mnk(M, N, K, 4);
  if (rc) return rc;
  return w4a8_call(M, N, K, x, wq, scales, zeros, y, ws, ws_bytes, true, stream, qg::W4A8_ASYM);
}

int qgemv_w4a8_noalloc(int M, int N, int K, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                       const uint32_t* zeros, uint16_t* y, qgemv_stream_t stream) {
  if (!x || !wq || !scales || !zeros || !y) return QGEMV_ERR_NULL;
  int rc = check_mnk(M, N, K, 4);
  if (rc) return rc;
  if ((size_t)M * K > QGEMV_W4A8_NOALLOC_MAX_MK) return QGEMV_ERR_WORKSPACE;
  void* ws = nullptr;
  rc = hip_status(qg::w4a8_noalloc_scratch(&ws));
  if (rc) return rc;
  return w4a8_call(M, N, K, x, wq, scales, zeros, y, ws, qg::w4a8_noalloc_scratch_bytes(), false, stream);
}

int qgemv_gemm_uniform(int bits, int M, int N, int K, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                       const uint32_t* zeros, uint16_t* y, qgemv_stream_t stream) {
  if (!x || !wq || !scales || !zeros || !y) return QGEMV_ERR_NULL;
  if (!valid_bits(bits)) return QGEMV_ERR_UNSUPPORTED;
  if (M < 1 || (M + 63) / 64 > 65535) return QGEMV_ERR_SHAPE;
  int rc = check_mnk(1, N, K, bits);
  if (rc) return rc;
  const long lim = 1L << 31;
  if ((long)M * K * 2 >= lim || (long)M * N * 2 >= lim) return QGEMV_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(wq) || ((uintptr_t)scales & 1u) || ((uintptr_t)zeros & 3u) ||
      ((uintptr_t)y & 1u))
    return QGEMV_ERR_ALIGN;
  const size_t ybytes = (size_t)M * N * 2;
  const int G = K / QGEMV_GROUP;
  if (overlaps(y, ybytes, x, (size_t)M * K * 2) ||
      overlaps(y, ybytes, wq, words(bits, QGEMV_LAYOUT_DEVICE, N, K) * 4) ||
      overlaps(y, ybytes, scales, (size_t)N * G * 2) ||
      overlaps(y, ybytes, zeros, words(bits, QGEMV_LAYOUT_PLAIN, N, G) * 4))
    return QGEMV_ERR_VALUE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Batch-size policy.  Up to 16 rows, the decode kernel; up to 64 rows,
  // whichever of the decode kernel on each 16-row slice and the GEMM the
  // cost model below prefers; beyond, the GEMM.
  const char* force = tune_env("QGEMV_GEMM_KERNEL");  // tuning override: "1" GEMM, "2" slices (M <= 64)
  const bool slices = force && force[0] == '1'   ? false
                      : force && force[0] == '2' ? M <= QGEMV_GEMM_SLICE_MAX_M
                                                 : prefer_slices(bits, M, N, K);
  if (slices) {
    for (int m0 = 0; m0 < M; m0 += QGEMV_MAX_M) {
      const int mm = M - m0 < QGEMV_MAX_M ? M - m0 : QGEMV_MAX_M;
      qg::UniformArgs a{bits, mm, N, K, x + (size_t)m0 * K, wq, scales, zeros, y + (size_t)m0 * N};
      rc = hip_status(qg::launch_gemv_tiles(a, tile_cfg(bits, mm, N, K, mm > 1), s));
      if (rc) return rc;
    }
    return QGEMV_OK;
  }
  qg::UniformArgs a{bits, M, N, K, x, wq, scales, zeros, y};
  int mi, nt, kh;
  gemm_block(bits, M, N, mi, nt, kh);
  if (const char* e = tune_env("QGEMV_GEMM_MI")) mi = std::atoi(e);  // tuning overrides
  if (const char* e = tune_env("QGEMV_GEMM_NT")) nt = std::atoi(e);
  if (const char* e = tune_env("QGEMV_GEMM_KH")) kh = std::atoi(e);
  if (kh == 2 && (nt != 2 || G % 2)) kh = 1;  // (two K halves: 128-column blocks, K/128 even)
  return hip_status(qg::launch_gemm_tiles(a, mi, nt, kh, s));
}

int qgemv_w2a16(int M, int N, int K, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                const uint32_t* zeros, uint16_t* y, qgemv_stream_t stream) {
  return qgemv_uniform(2, QGEMV_PATH_AUTO, M, N, K, x, wq, scales, zeros, y, stream);
}
int qgemv_w4a16(int M, int N, int K, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                const uint32_t* zeros, uint16_t* y, qgemv_stream_t stream) {
  return qgemv_uniform(4, QGEMV_PATH_AUTO, M, N, K, x, wq, scales, zeros, y, stream);
}
int qgemv_w8a16(int M, int N, int K, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                const uint32_t* zeros, uint16_t* y, qgemv_stream_t stream) {
  return qgemv_uniform(8, QGEMV_PATH_AUTO, M, N, K, x, wq, scales, zeros, y, stream);
}

int qgemv_outlier(int path, int M, int N, int K, const uint16_t* x, const uint32_t* wq, const uint16_t* scales,
                  const uint32_t* zeros, const uint32_t* tile_ptr, const uint32_t* tile_rec, int64_t nnz, uint16_t* y,
                  qgemv_stream_t stream) {
  if (!x || !wq || !scales || !zeros || !tile_ptr || !y || (nnz > 0 && !tile_rec)) return QGEMV_ERR_NULL;
  if (path != QGEMV_PATH_AUTO && path != QGEMV_PATH_VALU && path != QGEMV_PATH_MFMA)
    return QGEMV_ERR_UNSUPPORTED;
  int rc = check_mnk(M, N, K, 4);
  if (rc) return rc;
  if (nnz < 0 || nnz > (int64_t)N * K || nnz * 4 >= (int64_t)1 << 31) return QGEMV_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(wq) || ((uintptr_t)scales & 1u) || ((uintptr_t)zeros & 3u) ||
      ((uintptr_t)tile_ptr & 3u) || ((uintptr_t)tile_rec & 3u) || ((uintptr_t)y & 1u))
    return QGEMV_ERR_ALIGN;
  const size_t ybytes = (size_t)M * N * 2;
  const int G = K / QGEMV_GROUP;
  if (overlaps(y, ybytes, x, (size_t)M * K * 2) ||
      overlaps(y, ybytes, wq, words(4, QGEMV_LAYOUT_DEVICE, N, K) * 4) ||
      overlaps(y, ybytes, scales, (size_t)N * G * 2) ||
      overlaps(y, ybytes, zeros, words(4, QGEMV_LAYOUT_PLAIN, N, G) * 4) ||
      overlaps(y, ybytes, tile_ptr, qgemv_tilecoo_ptr_len(N, K) * 4) ||
      (nnz > 0 && overlaps(y, ybytes, tile_rec, (size_t)nnz * 4)))
    return QGEMV_ERR_VALUE;
  qg::UniformArgs a{4, M, N, K, x, wq, scales, zeros, y, tile_ptr, tile_rec, (int)nnz};
  if (path == QGEMV_PATH_AUTO) path = auto_path(4, M, N);
  const bool mfma = path == QGEMV_PATH_MFMA;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Wide layers (N >= 16384) at M >= 4: the fused kernel is held to two
  // tile-rows per workgroup there, and the dense kernel followed by the
  // separate sparse kernel is faster (28672 x 4096: 26.1 vs 37.4 us at M = 4,
  // 69.8 vs 83.3 at M = 16).  QGEMV_OUTLIER_FORM=fused|split forces a form.
  bool split = M >= 4 && N >= 16384 && K <= QGEMV_SPMV_MAX_K && (long)M * K * 2 + 512 < 1L << 31;
  if (const char* e = tune_env("QGEMV_OUTLIER_FORM")) split = std::strcmp(e, "split") == 0;
  if (split && !tune_env("QGEMV_OUTLIER_CFG")) {
    const qg::UniformArgs d{4, M, N, K, x, wq, scales, zeros, y, nullptr, nullptr, 0};
    const hipError_t e = qg::launch_gemv_tiles(d, tile_cfg(4, M, N, K, mfma), s);
    if (e != hipSuccess || nnz == 0) return hip_status(e);
    const qg::SpmvArgs sa{M, N, K, x, tile_ptr, tile_rec, (int)nnz, y};
    return hip_status(qg::launch_spmv_tilecoo(sa, s));
  }
  qg::TileCfg c = qg::pick_outlier(M, N, K, mfma);
  if (const char* e = tune_env("QGEMV_OUTLIER_CFG")) {  // tuning override "tpw,wk[,mt[,v]]"
    int tpw, wk, mt, v;
    const int n = std::sscanf(e, "%d,%d,%d,%d", &tpw, &wk, &mt, &v);
    if (n >= 2) {
      c.v = tpw != 1 ? 0 : (c.tpw == 1 ? c.v : 3);  // (a one-tile-row pick keeps its ring)
      c.tpw = tpw;
      c.wk = wk;
    }
    if (n >= 3 && !mfma) c.mt = mt;
    if (n >= 4) c.v = v;
  }
  return hip_status(qg::launch_gemv_outlier(a, c, s));
}

size_t qgemv_codebook_workspace_bytes(int M, int N, int K) {
  if (M < 1 || M > QGEMV_MAX_M || N < 1 || K < 512 || K % 512) return 0;
  return qg::codebook_ws_bytes(qg::pick_codebook(M, N, K), M, N, K);
}

int qgemv_codebook(int M, int N, int K, const uint16_t* x, const uint32_t* codes, const uint16_t* codebook,
                   const uint16_t* scales, uint16_t* y, void* ws, size_t ws_bytes, qgemv_stream_t stream) {
  if (!x || !codes || !codebook || !scales || !y) return QGEMV_ERR_NULL;
  if (M < 1 || M > QGEMV_MAX_M || N < 1 || K < 512 || K % 512) return QGEMV_ERR_SHAPE;
  const long lim = 1L << 31;
  if ((long)((N + 63) / 64) * 64 * (K / 4) >= lim || (long)M * K * 2 >= lim || (long)M * N * 2 >= lim)
    return QGEMV_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || ((uintptr_t)codebook & 3u) || ((uintptr_t)scales & 1u) ||
      ((uintptr_t)y & 1u) || ((uintptr_t)ws & 3u))
    return QGEMV_ERR_ALIGN;
  const size_t ybytes = (size_t)M * N * 2;
  if (overlaps(y, ybytes, x, (size_t)M * K * 2) ||
      overlaps(y, ybytes, codes, words(8, QGEMV_LAYOUT_ROWS64, N, K / 4) * 4) ||
      overlaps(y, ybytes, codebook, 256 * 4 * 2) || overlaps(y, ybytes, scales, (size_t)N * (K / 128) * 2) ||
      (ws && overlaps(y, ybytes, ws, ws_bytes)))
    return QGEMV_ERR_VALUE;
  if (ws && (overlaps(ws, ws_bytes, x, (size_t)M * K * 2) ||
             overlaps(ws, ws_bytes, codes, words(8, QGEMV_LAYOUT_ROWS64, N, K / 4) * 4) ||
             overlaps(ws, ws_bytes, codebook, 256 * 4 * 2) || overlaps(ws, ws_bytes, scales, (size_t)N * (K / 128) * 2)))
    return QGEMV_ERR_VALUE;
  qg::CodebookCfg c = qg::pick_codebook(M, N, K);
  // tuning override: "1,wk,pp,r[,mb]" (stationary) or "0,wk,ks" (sequential)
  if (const char* e = tune_env("QGEMV_CODEBOOK_CFG")) {
    int kind, wk, p1, p2 = 0, p3 = 1;
    if (std::sscanf(e, "%d,%d,%d,%d,%d", &kind, &wk, &p1, &p2, &p3) >= 3) {
      c.wk = wk;
      if (kind == 1) {
        c.pp = p1;
        c.r = p2;
        c.ks = 1;
        c.mb = p3;
      } else {
        c.pp = 0;
        c.r = 0;
        c.ks = p1;
        c.mb = 1;
      }
    }
  }
  const size_t need = qg::codebook_ws_bytes(c, M, N, K);
  if (need > 0 && (!ws || ws_bytes < need)) c = qg::codebook_fallback();  // no room for partial sums
  qg::CodebookArgs a{M, N, K, x, codes, codebook, scales, y, reinterpret_cast<float*>(ws)};
  return hip_status(qg::launch_gemv_codebook(a, c, reinterpret_cast<hipStream_t>(stream)));
}

namespace {
bool gen_format_ok(int ncb, int v, int group) {
  return (v == 4 || v == 8 || v == 16) && ncb >= 1 && ncb <= v / 4 && (group == 32 || group == 64 || group == 128);
}
}  // namespace

size_t qgemv_codebook_gen_workspace_bytes(int M, int N, int K, int ncb, int v, int group) {
  if (!gen_format_ok(ncb, v, group) || M < 1 || M > QGEMV_MAX_M || N < 1 || K < 256 || K % 256) return 0;
  return qg::codebook_gen_ws_bytes(M, N, K);
}

int qgemv_codebook_gen(int M, int N, int K, int ncb, int v, int group, const uint16_t* x, const uint32_t* codes,
                       const uint16_t* codebooks, const uint16_t* scales, uint16_t* y, void* ws, size_t ws_bytes,
                       qgemv_stream_t stream) {
  if (!x || !codes || !codebooks || !scales || !y) return QGEMV_ERR_NULL;
  if (!gen_format_ok(ncb, v, group)) return QGEMV_ERR_UNSUPPORTED;
  if (M < 1 || M > QGEMV_MAX_M || N < 1 || K < 256 || K % 256) return QGEMV_ERR_SHAPE;
  const size_t plane = words(8, QGEMV_LAYOUT_ROWS64, N, K / v) * 4;
  const long lim = 1L << 31;
  if ((long)(plane * ncb) >= lim || (long)M * K * 2 >= lim || (long)M * N * 2 >= lim ||
      (long)N * (K / group) * 2 >= lim)
    return QGEMV_ERR_SHAPE;
  if (!aligned16(codes) || ((uintptr_t)x & 7u) || ((uintptr_t)codebooks & 7u) || ((uintptr_t)scales & 1u) ||
      ((uintptr_t)y & 1u) || ((uintptr_t)ws & 3u))
    return QGEMV_ERR_ALIGN;
  const size_t ybytes = (size_t)M * N * 2, cbytes = (size_t)ncb * 256 * v * 2;
  const size_t xbytes = (size_t)M * K * 2, sbytes = (size_t)N * (K / group) * 2;
  if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, codes, plane * ncb) ||
      overlaps(y, ybytes, codebooks, cbytes) || overlaps(y, ybytes, scales, sbytes) ||
      (ws && overlaps(y, ybytes, ws, ws_bytes)))
    return QGEMV_ERR_VALUE;
  if (ws && (overlaps(ws, ws_bytes, x, xbytes) || overlaps(ws, ws_bytes, codes, plane * ncb) ||
             overlaps(ws, ws_bytes, codebooks, cbytes) || overlaps(ws, ws_bytes, scales, sbytes)))
    return QGEMV_ERR_VALUE;
  int ks = qg::codebook_gen_ks(M, N, K);
  if (const char* e = tune_env("QGEMV_CODEBOOK_GEN_KS")) {  // tuning override: K parts, or -wk (stationary)
    const int k = std::atoi(e);
    if (k >= 1) ks = k < K / 256 ? k : K / 256;
    if (k <= -1 && k >= -4) ks = k;
  }
  const size_t need = ks < 0 ? (size_t)(K / 256) * M * N * 4 : (ks > 1 ? (size_t)ks * M * N * 4 : 0);
  if (need > 0 && (!ws || ws_bytes < need)) ks = 1;  // no room for partial sums: one K range per workgroup
  qg::CodebookGenArgs a{M, N, K, ncb, v, group, x, codes, codebooks, scales, y, reinterpret_cast<float*>(ws)};
  return hip_status(qg::launch_gemv_codebook_gen(a, ks, reinterpret_cast<hipStream_t>(stream)));
}

int qgemv_lut4(int M, int N, int K, const uint16_t* x, const uint32_t* wq, const uint16_t* absmax,
               const uint16_t* lut, uint16_t* y, qgemv_stream_t stream) {
  if (!x || !wq || !absmax || !lut || !y) return QGEMV_ERR_NULL;
  int rc = check_mnk(M, N, K, 4);
  if (rc) return rc;
  if (K > QGEMV_LUT4_MAX_K || (size_t)K > qg::lut4_max_k(1)) return QGEMV_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(wq) || ((uintptr_t)absmax & 1u) || ((uintptr_t)lut & 1u) ||
      ((uintptr_t)y & 1u))
    return QGEMV_ERR_ALIGN;
  const size_t ybytes = (size_t)M * N * 2;
  if (overlaps(y, ybytes, x, (size_t)M * K * 2) ||
      overlaps(y, ybytes, wq, words(4, QGEMV_LAYOUT_DEVICE, N, K) * 4) ||
      overlaps(y, ybytes, absmax, (size_t)N * (K / QGEMV_LUT_BLOCK) * 2) || overlaps(y, ybytes, lut, 32))
    return QGEMV_ERR_VALUE;
  qg::Lut4Args a{M, N, K, x, wq, absmax, lut, y};
  return hip_status(qg::launch_gemv_lut4(a, lut4_cfg(M, N, K), reinterpret_cast<hipStream_t>(stream)));
}

// ---- unfused baselines ----

namespace {
int check_nk(int N, int K) {
  if (N < 1 || K < QGEMV_GROUP || K % QGEMV_GROUP) return QGEMV_ERR_SHAPE;
  if ((long)N * K * 2 >= 1L << 31 || (long)((N + 15) / 16) * 16 * K >= 1L << 31) return QGEMV_ERR_SHAPE;
  return QGEMV_OK;
}
}  // namespace

int qgemv_dequant(int bits, int N, int K, const uint32_t* wq, const uint16_t* scales, const uint32_t* zeros,
                  uint16_t* w, qgemv_stream_t stream) {
  if (!wq || !scales || !zeros || !w) return QGEMV_ERR_NULL;
  if (!valid_bits(bits)) return QGEMV_ERR_UNSUPPORTED;
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (!aligned16(wq) || !aligned16(w) || ((uintptr_t)scales & 1u) || ((uintptr_t)zeros & 3u))
    return QGEMV_ERR_ALIGN;
  const size_t wbytes = (size_t)N * K * 2;
  const int G = K / QGEMV_GROUP;
  if (overlaps(w, wbytes, wq, words(bits, QGEMV_LAYOUT_DEVICE, N, K) * 4) ||
      overlaps(w, wbytes, scales, (size_t)N * G * 2) ||
      overlaps(w, wbytes, zeros, words(bits, QGEMV_LAYOUT_PLAIN, N, G) * 4))
    return QGEMV_ERR_VALUE;
  qg::DequantArgs a{bits, N, K, wq, scales, zeros, nullptr, nullptr, w};
  return hip_status(qg::launch_dequant_uniform(a, reinterpret_cast<hipStream_t>(stream)));
}

int qgemv_dequant_lut4(int N, int K, const uint32_t* wq, const uint16_t* absmax, const uint16_t* lut, uint16_t* w,
                       qgemv_stream_t stream) {
  if (!wq || !absmax || !lut || !w) return QGEMV_ERR_NULL;
  int rc = check_nk(N, K);
  if (rc) return rc;
  if (!aligned16(wq) || !aligned16(w) || ((uintptr_t)absmax & 1u) || ((uintptr_t)lut & 1u))
    return QGEMV_ERR_ALIGN;
  const size_t wbytes = (size_t)N * K * 2;
  if (overlaps(w, wbytes, wq, words(4, QGEMV_LAYOUT_DEVICE, N, K) * 4) ||
      overlaps(w, wbytes, absmax, (size_t)N * (K / QGEMV_LUT_BLOCK) * 2) || overlaps(w, wbytes, lut, 32))
    return QGEMV_ERR_VALUE;
  qg::DequantArgs a{4, N, K, wq, nullptr, nullptr, absmax, lut, w};
  return hip_status(qg::launch_dequant_lut4(a, reinterpret_cast<hipStream_t>(stream)));
}

int qgemv_gemv_f16(int M, int N, int K, const uint16_t* x, const uint16_t* w, uint16_t* y,
                   qgemv_stream_t stream) {
  if (!x || !w || !y) return QGEMV_ERR_NULL;
  if (M < 1 || M > QGEMV_MAX_M) return QGEMV_ERR_SHAPE;
  int rc = check_nk(N, K);
  if (rc) return rc;
  if ((long)M * K * 2 >= 1L << 31) return QGEMV_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(w) || ((uintptr_t)y & 1u)) return QGEMV_ERR_ALIGN;
  const size_t ybytes = (size_t)M * N * 2;
  if (overlaps(y, ybytes, x, (size_t)M * K * 2) || overlaps(y, ybytes, w, (size_t)N * K * 2))
    return QGEMV_ERR_VALUE;
  qg::DenseCfg c = qg::pick_dense(M, N, K);
  if (const char* e = tune_env("QGEMV_DENSE_CFG")) {  // tuning override "tpw,s,wk"
    int tpw, st, wk;
    if (std::sscanf(e, "%d,%d,%d", &tpw, &st, &wk) == 3) c = {tpw, st, wk};
  }
  qg::DenseArgs a{M, N, K, x, w, y};
  return hip_status(qg::launch_gemv_f16(a, c, reinterpret_cast<hipStream_t>(stream)));
}

int qgemv_spmv_tilecoo(int M, int N, int K, const uint16_t* x, const uint32_t* tile_ptr, const uint32_t* tile_rec,
                       int64_t nnz, uint16_t* y, qgemv_stream_t stream) {
  if (!x || !tile_ptr || !y || (nnz > 0 && !tile_rec)) return QGEMV_ERR_NULL;
  if (M < 1 || M > QGEMV_MAX_M || N < 1 || K < QGEMV_GROUP || K % QGEMV_GROUP || K > QGEMV_SPMV_MAX_K)
    return QGEMV_ERR_SHAPE;
  // x is read at k up to 255 past a tile's start, within the buffer's bounds check
  if ((long)M * K * 2 + 512 >= 1L << 31 || (long)M * N * 2 >= 1L << 31) return QGEMV_ERR_SHAPE;
  if (nnz < 0 || nnz > (int64_t)N * K || nnz * 4 >= (int64_t)1 << 31) return QGEMV_ERR_SHAPE;
  if (!aligned16(x) || ((uintptr_t)tile_ptr & 3u) || ((uintptr_t)tile_rec & 3u) || ((uintptr_t)y & 1u))
    return QGEMV_ERR_ALIGN;
  const size_t ybytes = (size_t)M * N * 2;
  if (overlaps(y, ybytes, x, (size_t)M * K * 2) || overlaps(y, ybytes, tile_ptr, qgemv_tilecoo_ptr_len(N, K) * 4) ||
      (nnz > 0 && overlaps(y, ybytes, tile_rec, (size_t)nnz * 4)))
    return QGEMV_ERR_VALUE;
  if (nnz == 0) return QGEMV_OK;  // nothing to add
  qg::SpmvArgs a{M, N, K, x, tile_ptr, tile_rec, (int)nnz, y};
  return hip_status(qg::launch_spmv_tilecoo(a, reinterpret_cast<hipStream_t>(stream)));
}

// ---- measurement ----

int qgemv_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, int threads,
                      qgemv_stream_t stream) {
  if (!src || !sink) return QGEMV_ERR_NULL;
  if (bytes == 0 || bytes % 16 || workgroups < 1 || threads < 64 || threads > 1024 || threads % 64)
    return QGEMV_ERR_SHAPE;
  if (!aligned16(src) || ((uintptr_t)sink & 3u)) return QGEMV_ERR_ALIGN;
  if (overlaps(sink, 4, src, bytes)) return QGEMV_ERR_VALUE;
  return hip_status(qg::launch_stream_read(src, bytes, sink, workgroups, threads,
                                           reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
