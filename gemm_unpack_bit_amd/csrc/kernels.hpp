// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

// A tuning override from the environment, or NULL: looked up only when
// QGEMV_TUNING was set at the process's first call (api.cpp).
const char* tune_env(const char* name);

struct UniformArgs {
  int bits, M, N, K;
  const uint16_t* x;
  const uint32_t* wq;
  const uint16_t* scales;
  const uint32_t* zeros;
  uint16_t* y;
  // outlier variant only (nullptr / 0 otherwise): Tile-COO fp16 outliers
  const uint32_t* tile_ptr;
  const uint32_t* tile_rec;
  int nnz;
};

// Launch shape of the tiled kernel: mfma selects the dot engine; mt = batch
// rows per pass of the VALU engine (1 or 2; the MFMA engine takes all 16);
// tpw = 16-row tile-rows per workgroup (1 [v = 3 only], 2, 4, 8); wk = waves per workgroup,
// which take the chunks of quant groups round-robin (1..8, 16 for one-group
// chunks); v = pipeline
// variant (0: 4-group chunks, 2 stage buffers; 1: 2-group chunks, 4 buffers;
// tpw must be a multiple of the buffer count).
struct TileCfg {
  bool mfma;
  int mt, tpw, wk, v;
  bool xd = false;  // matrix-core engine, activations not staged whole: the per-wave activation ring
};

TileCfg pick_tiles(int bits, int M, int N, int K, bool mfma);
hipError_t launch_gemv_tiles(const UniformArgs& a, const TileCfg& c, hipStream_t s);
// W4 dense + Tile-COO sparse in one kernel (tpw 1 with v 3, or tpw 2 with v 0)
TileCfg pick_outlier(int M, int N, int K, bool mfma);
hipError_t launch_gemv_outlier(const UniformArgs& a, const TileCfg& c, hipStream_t s);

// 4-bit codes (tiled device layout) with a 16-entry fp16 table and fp16
// per-64-block scales: y = x . (LUT[q] * absmax)^T
struct Lut4Args {
  int M, N, K;
  const uint16_t* x;
  const uint32_t* wq;
  const uint16_t* absmax;
  const uint16_t* lut;
  uint16_t* y;
};
// LUT4 launch: mt activation rows per workgroup (1, 2), tpw tile-rows per
// workgroup (1 with ng = 1, or 2 with ng = 4), ng groups per chunk, wk waves
// (1..8), d chunks in each wave's ring (tpw 1 only)
struct Lut4Cfg {
  int mt, tpw, ng, wk, d;
};
Lut4Cfg pick_lut4(int M, int N, int K);
size_t lut4_max_k(int mt);  // largest K the LDS staging holds at mt rows
hipError_t launch_gemv_lut4(const Lut4Args& a, const Lut4Cfg& c, hipStream_t s);

// Codebook (m = 1, v = 4, b = 8, g = 128) with a Psumbook: codes [N, K/4]
// uint8 in the 64-row layout (layout 2), codebook fp16 [256][4], scales fp16
// [N, K/128]; ws: the K-split partial sums (KS x M x N fp32)
struct CodebookArgs {
  int M, N, K;
  const uint16_t* x;
  const uint32_t* codes;
  const uint16_t* codebook;
  const uint16_t* scales;
  uint16_t* y;
  float* ws;
};
// A codebook launch.  pp > 0 (1, 2, 4): the stationary kernel, one K part of pp pairs
// (256 k each) per workgroup and r row slices, its Psumbook entries holding mb
// batch rows (1, 2, 4; pp * mb <= 4); pp == 0: the sequential kernel, ks K
// ranges per row block (ks == 1 needs no workspace).  wk = waves per
// workgroup (1, 2, 4, 8, 16).
struct CodebookCfg {
  int wk, pp, r, ks, mb;
};
CodebookCfg pick_codebook(int M, int N, int K);
CodebookCfg codebook_fallback();
size_t codebook_ws_bytes(const CodebookCfg& c, int M, int N, int K);
hipError_t launch_gemv_codebook(const CodebookArgs& a, const CodebookCfg& c, hipStream_t s);

// General codebook kernel: ncb additive codebooks [ncb][256][v] fp16 (v = 4,
// 8, 16; ncb <= v / 4), codes as ncb planes of [N, K/v] uint8 in the 64-row
// layout, scales fp16 [N, K/group] (group = 32, 64, 128); ws: the K parts'
// fp32 partial sums (ks x M x N) when ks > 1
struct CodebookGenArgs {
  int M, N, K, ncb, v, group;
  const uint16_t* x;
  const uint32_t* codes;
  const uint16_t* codebooks;
  const uint16_t* scales;
  uint16_t* y;
  float* ws;
};
int codebook_gen_ks(int M, int N, int K);
size_t codebook_gen_ws_bytes(int M, int N, int K);
// ks >= 1: the sequential form with ks K parts; ks = -wk: the stationary
// form with wk (1..4) waves per workgroup (one K part per 256-k chunk)
hipError_t launch_gemv_codebook_gen(const CodebookGenArgs& a, int ks, hipStream_t s);

// W4A8 with the padding strategy (gemv_w4a8.hip): int8 activations per row
// in the workspace (xq [M, K], then sx [M] fp32 at a 16-byte boundary)
// W4A8 strategies: padding (int8 matrix cores, symmetric activations),
// split (the int8 activations in two 4-bit slices on the fp8 matrix cores)
// and asymmetric activations (zero points on both operands, int8 matrix
// cores on the raw codes, zero-point expansion)
enum W4A8Mode { W4A8_PAD = 0, W4A8_SPLIT = 1, W4A8_ASYM = 2 };
struct W4A8Args {
  int M, N, K;
  const uint16_t* x;
  const uint32_t* wq;
  const uint16_t* scales;
  const uint32_t* zeros;
  uint16_t* y;
  int8_t* xq;   // pad, asym: int8 activations [M, K]; split: 16 h as fp8 [M, K]
  float* sx;    // activation scales [M]
  int mode;     // W4A8Mode
  uint8_t* xl;  // split: the low slices l as fp8 [M, K]
  int* zx;      // asym: activation zero points [16]
  int* xsum;    // asym: per-group sums of the int8 activations [K/128][16]
};
// workspace layout of each mode: the byte offsets of xq, xl, sx, zx, xsum
// and the total (unused parts 0)
struct W4A8Ws {
  size_t xq, xl, sx, zx, xsum, total;
};
W4A8Ws w4a8_ws_layout(int mode, int M, int K);
size_t w4a8_ws_bytes(int M, int K);
// qgemv_w4a8_noalloc: largest M * K its static scratch holds, the scratch's
// size, and its device address on the current device (looked up once per
// device)
constexpr size_t W4A8_NOALLOC_MAX_MK = 1u << 20;
size_t w4a8_noalloc_scratch_bytes();
hipError_t w4a8_noalloc_scratch(void** ptr);
int w4a8_waves(int N, int K);
hipError_t launch_gemv_w4a8(const W4A8Args& a, int wk, hipStream_t s);

// Prefill-size GEMM (gemm_tiles.hip): the uniform format at any M on the
// matrix cores, blocks of 16 mi activation rows (mi = 2, 4) x 64 nt weight
// rows (nt = 2, 4), K split in kh halves inside the workgroup (kh = 2: nt = 2
// and K/128 even only)
hipError_t launch_gemm_tiles(const UniformArgs& a, int mi, int nt, int kh, hipStream_t s);

// Unfused baselines (unfused.hip): eager dequantization to fp16 W [N, K]
// row-major (uniform b-bit: bits, wq, scales, zeros; LUT4: wq, absmax, lut),
// a dense fp16 GEMV over it, and a Tile-COO SpMV that adds x . S^T into y.
struct DequantArgs {
  int bits, N, K;
  const uint32_t* wq;
  const uint16_t* scales;
  const uint32_t* zeros;
  const uint16_t* absmax;
  const uint16_t* lut;
  uint16_t* w;
};
hipError_t launch_dequant_uniform(const DequantArgs& a, hipStream_t s);
hipError_t launch_dequant_lut4(const DequantArgs& a, hipStream_t s);

struct DenseArgs {
  int M, N, K;
  const uint16_t* x;
  const uint16_t* w;
  uint16_t* y;
};
// tpw row tiles of 16 per workgroup, s MFMA k-steps (32 k each) per chunk,
// wk waves: (1, 8), (1, 4), (2, 4) or (4, 4) with wk 1..8
struct DenseCfg {
  int tpw, s, wk;
};
DenseCfg pick_dense(int M, int N, int K);
hipError_t launch_gemv_f16(const DenseArgs& a, const DenseCfg& c, hipStream_t s);

struct SpmvArgs {
  int M, N, K;
  const uint16_t* x;
  const uint32_t* tile_ptr;
  const uint32_t* tile_rec;
  int nnz;
  uint16_t* y;
};
size_t spmv_lds_bytes(int K);
hipError_t launch_spmv_tilecoo(const SpmvArgs& a, hipStream_t s);

// bit packing (layout: 0 plain, 1 device = tiled, see pack.hip)
// streaming-read probe (measurement): reads `bytes` (a multiple of 16) once
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, int threads,
                              hipStream_t s);

size_t packed_words(int bits, int layout, int rows, int cols);
hipError_t launch_pack(int bits, int layout, int rows, int cols, const uint8_t* codes, uint32_t* packed,
                       hipStream_t s);
hipError_t launch_unpack(int bits, int layout, int rows, int cols, const uint32_t* packed, uint8_t* codes,
                         hipStream_t s);
// reads and clears the pack kernel's out-of-range flag (synchronizes s)
hipError_t pack_error_flag(int* flag, hipStream_t s);

}  // namespace qg
