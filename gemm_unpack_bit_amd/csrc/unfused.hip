// Unfused baselines of the quantized GEMV: the kernel sequences the fused
// kernels are measured against.
//
//  * Eager dequantization (Fast NF4 Dequantization Kernels page, method: the
//    codes are read from global memory, turned into fp16 on chip and written
//    back for a separate matrix product; QFactory review, "Problem and
//    motivation": eager execution dequantizes every element on its own):
//    dequant_tiles_kernel (uniform b-bit groups) and dequant_lut4_kernel
//    (16-entry table, per-64 block scale) write fp16 W [N, K] row-major;
//    gemv_f16_kernel then computes y = x . W^T from it.
//  * A separate sparse kernel for the outliers (FlashQuant abstract: existing
//    outlier-aware implementations run the low-bit dense path and the fp16
//    sparse path in two kernels that share activations and outputs):
//    spmv_tilecoo_kernel adds x . S^T into the y that the dense kernel wrote.
//
// Every result is deterministic: fixed summation orders, no atomics.
#include "common.hpp"
#include "dequant.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

// ---------------------------------------------------------------------------
// Eager dequantization.  One wave per 16 x 128 tile of the device layout:
// lane l owns row 16 rt + l % 16 and the 32 k of quarter l / 16.  The unpack
// gives q - z exactly in fp16 and one packed fp16 multiply by the group scale
// rounds the exact product s (q - z) once, to nearest even.
// ---------------------------------------------------------------------------
constexpr int DQ_WAVES = 4;  // waves (tiles) per workgroup
constexpr int DQ_ROW = 136;  // halves per staged tile row: 128 + 8 of padding (bank spread)

__device__ __forceinline__ void wave_lds_sync() {  // the wave's own LDS writes done
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt 0
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Write a dequantized 16 x 128 tile: lane l holds o[0..3] = row l % 16, k
// [32 (l / 16), +32).  Passed through the wave's LDS slot so that each store
// instruction writes 4 whole rows of the tile (4 x 256 contiguous bytes)
// instead of 16 scattered 64-byte pieces (whole lines, so non-temporal
// stores stream them to memory).
__device__ __forceinline__ void store_tile(const u4 (&o)[4], _Float16* slot, uint16_t* w, int N, int K, int rt,
                                           int g) {
  const int lane = threadIdx.x & 63;
  u4* sl = reinterpret_cast<u4*>(slot + (lane & 15) * DQ_ROW + 32 * (lane >> 4));
#pragma unroll
  for (int v = 0; v < 4; ++v) sl[v] = o[v];
  wave_lds_sync();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * j + (lane >> 4);
    const u4 v = *reinterpret_cast<const u4*>(slot + r * DQ_ROW + 8 * (lane & 15));
    const int n = 16 * rt + r;
    if (n < N) __builtin_nontemporal_store(v, reinterpret_cast<u4*>(w + (size_t)n * K + 128 * g + 8 * (lane & 15)));
  }
}

template <int BITS>
__global__ void __launch_bounds__(64 * DQ_WAVES) dequant_tiles_kernel(DequantArgs a) {
  constexpr int P = 32 / BITS;   // codes per word
  constexpr int NW = BITS;       // words per lane
  __shared__ __align__(16) _Float16 stage[DQ_WAVES][16 * DQ_ROW];
  const int lane = threadIdx.x & 63;
  const int G = a.K / 128;
  const uint32_t tile = blockIdx.x * DQ_WAVES + (threadIdx.x >> 6);
  if (tile >= (uint32_t)((a.N + 15) / 16) * G) return;  // (no workgroup barrier below)
  const int rt = (int)(tile / G), g = (int)(tile % G);
  const int n = 16 * rt + (lane & 15);

  const uint32_t tb = tile * 256u * BITS;  // tile byte offset
  const rsrc_t rw = make_rsrc(a.wq, (uint32_t)((a.N + 15) / 16) * 16u * a.K * BITS / 8u);
  uint32_t w[NW];
  if constexpr (BITS == 2) {
    const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rw, tb + 8u * lane, 0, CPOL_NT));
    w[0] = v.x;
    w[1] = v.y;
  } else {
#pragma unroll
    for (int h = 0; h < NW / 4; ++h) {
      const u4 v = bload16<CPOL_NT>(rw, tb + 1024u * h + 16u * lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[4 * h + e] = v[e];
    }
  }
  // group scale and zero point of (n, g); rows past N read 0 (never stored)
  const int ZW = (G * BITS + 31) / 32;
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)a.N * G * 2u);
  const rsrc_t rz = make_rsrc(a.zeros, (uint32_t)a.N * ZW * 4u);
  const uint16_t sb = bload2(rs, ((uint32_t)n * G + g) * 2u);
  const uint32_t zw = bload4(rz, ((uint32_t)n * ZW + (g * BITS) / 32) * 4u);
  const uint32_t z = (zw >> ((g * BITS) & 31)) & ((1u << BITS) - 1u);

  const typename Uni<BITS>::Z zc = Uni<BITS>::zc(z);
  const uint32_t mg = magic1024x2();
  const _Float16 s = __builtin_bit_cast(_Float16, sb);
  const h2 s2 = {s, s};
  h2 o[NW * P / 2];  // the lane's 32 weights in k order
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    h2 d[P / 2];
    Uni<BITS>::deq(w[i], mg, zc, d);
#pragma unroll
    for (int j = 0; j < P / 2; ++j) o[i * (P / 2) + j] = d[j] * s2;
  }
  u4 ov[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) ov[v] = u4{as_u32(o[4 * v]), as_u32(o[4 * v + 1]), as_u32(o[4 * v + 2]), as_u32(o[4 * v + 3])};
  store_tile(ov, stage[threadIdx.x >> 6], a.w, a.N, a.K, rt, g);
}

// NF4-style codes: w = LUT[q] * absmax[n, k / 64].  A 256-entry LDS table maps
// a byte (code c0 in the low nibble, c1 in the high one) to the fp16 pair
// (LUT[c0], LUT[c1]); a word's byte indices for the pairs (k, k + 1) come from
// two masks and two shifts (fields f and f + 4 hold k = 2f and 2f + 1).
__global__ void __launch_bounds__(64 * DQ_WAVES) dequant_lut4_kernel(DequantArgs a) {
  __shared__ uint32_t tab[256];
  __shared__ __align__(16) _Float16 stage[DQ_WAVES][16 * DQ_ROW];
  const int lane = threadIdx.x & 63;
  {
    const rsrc_t rl = make_rsrc(a.lut, 32u);
    const uint32_t t = threadIdx.x;  // 256 threads, one entry each
    tab[t] = (uint32_t)bload2(rl, 2u * (t & 15u)) | ((uint32_t)bload2(rl, 2u * (t >> 4)) << 16);
  }
  __syncthreads();
  const int G = a.K / 128;
  const uint32_t tile = blockIdx.x * DQ_WAVES + (threadIdx.x >> 6);
  if (tile >= (uint32_t)((a.N + 15) / 16) * G) return;
  const int rt = (int)(tile / G), g = (int)(tile % G);
  const int n = 16 * rt + (lane & 15), kq = lane >> 4;
  const rsrc_t rw = make_rsrc(a.wq, (uint32_t)((a.N + 15) / 16) * 16u * a.K / 2u);
  const u4 wv = bload16<CPOL_NT>(rw, tile * 1024u + 16u * lane);
  // the lane's 32 k lie in one 64-block: block 2 g + kq / 2
  const int KB = a.K / 64;
  const rsrc_t ra = make_rsrc(a.absmax, (uint32_t)a.N * KB * 2u);
  const uint16_t ab = bload2(ra, ((uint32_t)n * KB + 2 * g + (kq >> 1)) * 2u);  // (0 past N)
  const _Float16 s = __builtin_bit_cast(_Float16, ab);
  const h2 s2 = {s, s};
  u4 ov[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wd = wv[i];
    const uint32_t t = wd & 0x0F0F0F0Fu, u = (wd >> 4) & 0x0F0F0F0Fu;
    const uint32_t v0 = t | (t >> 12);  // byte 0: fields 0, 4 (k 0, 1); byte 1: fields 2, 6 (k 4, 5)
    const uint32_t v1 = u | (u >> 12);  // byte 0: fields 1, 5 (k 2, 3); byte 1: fields 3, 7 (k 6, 7)
    const h2 e0 = as_h2(tab[v0 & 0xFFu]) * s2, e1 = as_h2(tab[v1 & 0xFFu]) * s2;
    const h2 e2 = as_h2(tab[(v0 >> 8) & 0xFFu]) * s2, e3 = as_h2(tab[(v1 >> 8) & 0xFFu]) * s2;
    ov[i] = u4{as_u32(e0), as_u32(e1), as_u32(e2), as_u32(e3)};
  }
  store_tile(ov, stage[threadIdx.x >> 6], a.w, a.N, a.K, rt, g);
}

// ---------------------------------------------------------------------------
// Dense fp16 GEMV y = x . W^T (W [N, K] row-major) on the matrix cores, for
// every M in 1..16: A = x (batch rows; rows past M read zeros), B = 16 weight
// rows x 32 k, so one v_mfma_f32_16x16x32_f16 covers 16 rows x 32 k.  Lane l
// loads x[l % 16][k + 8 (l / 16) ..] and W[n + l % 16][k + 8 (l / 16) ..]: both
// operands use the same lane-to-k assignment, so the contraction is exact up
// to fp32 rounding.  A workgroup owns TPW row tiles of 16; its waves take
// chunks of 32 S k round-robin, two chunks in flight; waves are summed
// through LDS in a fixed order.  k past K and rows past N read zeros.
// ---------------------------------------------------------------------------
template <int TPW, int S>
__global__ void __launch_bounds__(512) gemv_f16_kernel(DenseArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, WK = blockDim.x >> 6;
  const int r = lane & 15, kq = lane >> 4;
  const int K = a.K;
  constexpr int CK = 32 * S;
  const int NC = (K + CK - 1) / CK;
  const int n0 = blockIdx.x * 16 * TPW;
  const rsrc_t rw = make_rsrc(a.w, (uint32_t)a.N * K * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * K * 2u);
  uint32_t wo[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int row = n0 + 16 * t + r;
    wo[t] = row < a.N ? ((uint32_t)row * K + 8u * kq) * 2u : OOB;
  }
  const uint32_t xo = r < a.M ? ((uint32_t)r * K + 8u * kq) * 2u : OOB;

  struct St {
    u4 A[S];
    u4 B[TPW][S];
  };
  auto load = [&](int c, St& st) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const int kk = c * CK + 32 * s;
      const bool in = c < NC && kk < K;  // wave-uniform
      const uint32_t so = in ? 2u * kk : 0u;
      st.A[s] = bload16(rx, in ? xo : OOB, so);
#pragma unroll
      for (int t = 0; t < TPW; ++t) st.B[t][s] = bload16<CPOL_NT>(rw, in ? wo[t] : OOB, so);
    }
  };
  f4 acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const St& st) {
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int t = 0; t < TPW; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, st.A[s]),
                                                       __builtin_bit_cast(h8, st.B[t][s]), acc[t], 0, 0, 0);
  };
  St st0, st1;
  int c = wave;
  load(c, st0);
  for (; c < NC; c += 2 * WK) {  // chunks past the last read zeros and add nothing
    load(c + WK, st1);
    __builtin_amdgcn_sched_barrier(0);
    mma(st0);
    __builtin_amdgcn_sched_barrier(0);
    load(c + 2 * WK, st0);
    __builtin_amdgcn_sched_barrier(0);
    mma(st1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // lane l holds D[m = 4 (l / 16) + v][row l % 16] of each row tile
  f4* red = reinterpret_cast<f4*>(smem);
#pragma unroll
  for (int t = 0; t < TPW; ++t) red[(wave * TPW + t) * 64 + lane] = acc[t];
  __syncthreads();
  for (int e = threadIdx.x; e < TPW * 256; e += blockDim.x) {
    const int v = e & 3, l = (e >> 2) & 63, t = e >> 8;
    const int m = 4 * (l >> 4) + v, row = n0 + 16 * t + (l & 15);
    if (m >= a.M || row >= a.N) continue;
    float sum = 0.f;
    for (int w = 0; w < WK; ++w) sum += red[(w * TPW + t) * 64 + l][v];
    a.y[(size_t)m * a.N + row] = f2h(sum);
  }
}

// ---------------------------------------------------------------------------
// Separate Tile-COO SpMV: y[m, n] += sum over the outliers (n, k, v) of
// v x[m, k], on the y that the dense kernel wrote (one more fp16 rounding).
// One workgroup per 16-row tile-row; its records are one contiguous range
// (tiles in row-tile-major order).  Wave w takes batches w, w + WK, ... of 64
// records (the next batch's records in flight while one is processed): lane i
// reads record i, finds its tile by binary search over the tile-row's
// tile_ptr entries (staged in LDS), and stages its row and its products
// v x[m, k] in the wave's LDS slot.  Lane (row r, quarter p) then sums the
// products of the batch's quarter p whose row is r.  Quarters and waves are
// added in a fixed order; rows with no outlier keep their bits.  MB bounds the
// batch rows M (1, 2, 4, 8, 16).
// ---------------------------------------------------------------------------
constexpr int SP_WAVES = 4;

template <int MB>
__global__ void __launch_bounds__(64 * SP_WAVES) spmv_tilecoo_kernel(SpmvArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = a.K / 128, M = a.M;
  const int rt = blockIdx.x;
  float* part = reinterpret_cast<float*>(smem);                 // [SP_WAVES][17][16]: M sums + hit flag
  uint32_t* rowl = reinterpret_cast<uint32_t*>(part + SP_WAVES * 17 * 16) + wave * 64 * 17;  // [64] rows
  float* cs = reinterpret_cast<float*>(rowl + 64);              // [16][64] products
  uint32_t* ptr = reinterpret_cast<uint32_t*>(part + SP_WAVES * 17 * 16) + SP_WAVES * 64 * 17;  // [G + 1]
  const rsrc_t rp = make_rsrc(a.tile_ptr, ((uint32_t)((a.N + 15) / 16) * G + 1u) * 4u);
  for (int i = threadIdx.x; i <= G; i += blockDim.x) ptr[i] = bload4(rp, ((uint32_t)rt * G + i) * 4u);
  // thread e < 16 M owns output (m, n) = (e / 16, 16 rt + e % 16): its prior y, loaded early
  const int em = threadIdx.x >> 4, en = 16 * rt + (threadIdx.x & 15);
  const bool eo = em < M && en < a.N;
  const rsrc_t ry = make_rsrc(a.y, (uint32_t)M * a.N * 2u);
  const uint16_t yprior = bload2(ry, eo ? ((uint32_t)em * a.N + en) * 2u : OOB);
  __syncthreads();
  const uint32_t beg = ptr[0];
  const uint32_t end = min(ptr[G], beg + 2048u * (uint32_t)G);  // (a tile holds at most 2048 records)
  if (beg >= end) return;  // no outliers in this tile-row: y untouched
  const rsrc_t rr = make_rsrc(a.tile_rec, (uint32_t)a.nnz * 4u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * a.K * 2u);
  const int r = lane & 15, p = lane >> 4;
  const int top = 1 << (31 - __builtin_clz(G));  // largest power of two <= G
  float acc[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) acc[m] = 0.f;
  uint32_t hit = 0;
  uint32_t b0 = beg + 64u * wave;
  uint32_t rec_n = bload4(rr, b0 + lane < end ? 4u * (b0 + lane) : OOB);
  for (; b0 < end; b0 += 64u * SP_WAVES) {  // wave-uniform
    const uint32_t i = b0 + lane;
    const bool ok = i < end;
    const uint32_t rec = rec_n;
    const uint32_t inext = i + 64u * SP_WAVES;
    rec_n = bload4(rr, inext < end ? 4u * inext : OOB);
    int g = 0;  // the last tile whose range starts at or before record i
    for (int s = top; s > 0; s >>= 1)
      if (g + s < G && ptr[g + s] <= i) g += s;
    const uint32_t col = 128u * g + (rec & 0xFFu);
    const float v = h2f((uint16_t)(rec >> 16));
#pragma unroll
    for (int m = 0; m < MB; ++m)
      if (m < M) cs[m * 64 + lane] = v * h2f(bload2(rx, ok ? ((uint32_t)m * a.K + col) * 2u : OOB));
    rowl[lane] = ok ? (rec >> 8) & 0xFFu : 0xFFFFu;
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = 16 * p + j;
      if (rowl[e] == (uint32_t)r) {
        hit = 1;
#pragma unroll
        for (int m = 0; m < MB; ++m)
          if (m < M) acc[m] += cs[m * 64 + e];
      }
    }
    wave_lds_sync();  // the slot is rewritten by the next batch
  }
  // quarters (q0 + q2) + (q1 + q3), then waves in order
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    if (m < M) {
      const float sm = quarter_sum(acc[m]);
      if (p == 0) part[(wave * 17 + m) * 16 + r] = sm;
    }
  }
  const float hf = quarter_sum((float)hit);
  if (p == 0) part[(wave * 17 + 16) * 16 + r] = hf;
  __syncthreads();
  if (eo) {
    const int er = threadIdx.x & 15;
    float any = 0.f, sum = 0.f;
    for (int w = 0; w < SP_WAVES; ++w) {
      any += part[(w * 17 + 16) * 16 + er];
      sum += part[(w * 17 + em) * 16 + er];
    }
    if (any > 0.f) a.y[(size_t)em * a.N + en] = f2h(h2f(yprior) + sum);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_dequant_uniform(const DequantArgs& a, hipStream_t s) {
  const uint32_t tiles = (uint32_t)((a.N + 15) / 16) * (a.K / 128);
  const dim3 grid((tiles + DQ_WAVES - 1) / DQ_WAVES), block(64 * DQ_WAVES);
  switch (a.bits) {
    case 2: hipLaunchKernelGGL(dequant_tiles_kernel<2>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(dequant_tiles_kernel<4>, grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL(dequant_tiles_kernel<8>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequant_lut4(const DequantArgs& a, hipStream_t s) {
  const uint32_t tiles = (uint32_t)((a.N + 15) / 16) * (a.K / 128);
  hipLaunchKernelGGL(dequant_lut4_kernel, dim3((tiles + DQ_WAVES - 1) / DQ_WAVES), dim3(64 * DQ_WAVES), 0, s, a);
  return hipGetLastError();
}

// Fitted to sweeps of every shape on MI355X (Llama-3-8B layer shapes, M = 1,
// 4, 16; cache-cold): one row tile and 128-k chunks (80 VGPRs, so several
// workgroups share a CU), with the waves per workgroup set by the grid width
// -- 4 (8 for long K) when there are at most 256 row tiles, 2 up to 1024, 4
// beyond; from M = 9 on, 2 waves and two row tiles per workgroup on wide
// layers, which share each x fragment.
DenseCfg pick_dense(int M, int N, int K) {
  const int NT = (N + 15) / 16;
  DenseCfg c{1, 4, 4};
  if (M > 8) {
    c.wk = 2;
    if (NT >= 384) c.tpw = 2;
  } else if (NT <= 256) {
    c.wk = K >= 8192 ? 8 : 4;
  } else if (NT <= 1024) {
    c.wk = 2;
  }
  const int nc = (K + 32 * c.s - 1) / (32 * c.s);
  if (c.wk > nc) c.wk = nc;
  return c;
}

hipError_t launch_gemv_f16(const DenseArgs& a, const DenseCfg& c, hipStream_t s) {
  if (c.wk < 1 || c.wk > 8) return hipErrorInvalidValue;
  const int NT = (a.N + 15) / 16;
  const dim3 grid((NT + c.tpw - 1) / c.tpw), block(64 * c.wk);
  const size_t lds = (size_t)c.wk * c.tpw * 64 * 16;
  if (c.tpw == 1 && c.s == 8) hipLaunchKernelGGL((gemv_f16_kernel<1, 8>), grid, block, lds, s, a);
  else if (c.tpw == 1 && c.s == 4) hipLaunchKernelGGL((gemv_f16_kernel<1, 4>), grid, block, lds, s, a);
  else if (c.tpw == 2 && c.s == 4) hipLaunchKernelGGL((gemv_f16_kernel<2, 4>), grid, block, lds, s, a);
  else if (c.tpw == 4 && c.s == 4) hipLaunchKernelGGL((gemv_f16_kernel<4, 4>), grid, block, lds, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

size_t spmv_lds_bytes(int K) { return (size_t)SP_WAVES * 17 * 16 * 4 + (size_t)SP_WAVES * 64 * 17 * 4 + (size_t)(K / 128 + 1) * 4; }

hipError_t launch_spmv_tilecoo(const SpmvArgs& a, hipStream_t s) {
  const dim3 grid((a.N + 15) / 16), block(64 * SP_WAVES);
  const size_t lds = spmv_lds_bytes(a.K);
  if (a.M <= 1) hipLaunchKernelGGL(spmv_tilecoo_kernel<1>, grid, block, lds, s, a);
  else if (a.M <= 2) hipLaunchKernelGGL(spmv_tilecoo_kernel<2>, grid, block, lds, s, a);
  else if (a.M <= 4) hipLaunchKernelGGL(spmv_tilecoo_kernel<4>, grid, block, lds, s, a);
  else if (a.M <= 8) hipLaunchKernelGGL(spmv_tilecoo_kernel<8>, grid, block, lds, s, a);
  else hipLaunchKernelGGL(spmv_tilecoo_kernel<16>, grid, block, lds, s, a);
  return hipGetLastError();
}

}  // namespace qg
