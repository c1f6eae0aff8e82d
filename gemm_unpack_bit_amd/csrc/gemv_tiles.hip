// Fused dequantize-and-multiply for group-wise asymmetric WbA16 weights
// (b = 2, 4, 8) at decode batch M <= 16, on gfx950.
//
//   y[m, n] = sum_k x[m, k] * s[n, k/128] * (q[n, k] - z[n, k/128])
//
// The weight-only group-wise asymmetric format of the QFactory (ATC'25)
// review ("Problem and motivation"; "Experiments": asymmetric W8/W4/W2, group
// 128x1).  Two dot engines share one kernel body:
//  * VALU (batch 1-2): v_dot2_f32_f16 of the unpacked pairs with x into fp32
//    partials, one per lane, tile-row and batch row;
//  * MFMA (skinny GEMM, the regime where the pages report hand-written
//    matrix-core kernels overtaking bandwidth-only ones as batch grows --
//    QFactory review Table 3, ADAngel review observation 2): the unpacked pairs
//    are directly the B operand of v_mfma_f32_16x16x32_f16, x (M padded to 16
//    rows with zeros) the A operand, and the K reduction runs in the matrix core.
//
// Data path (both engines):
//  * Weights are in the tiled device layout: one 16-row x 128-k tile (one
//    quant group) is a contiguous block in which lane l holds row l % 16 and
//    the 32 consecutive k of quarter l / 16, and the tiles of a tile-row follow
//    each other along k.  Every wave-wide load is one contiguous 512 B..1 KB
//    burst, read once and non-temporal through raw buffer loads (out-of-range
//    rows and groups read zeros, so ragged edges need no branches).
//  * Work split: a workgroup owns TPW consecutive tile-rows (16*TPW weight
//    rows) and all of K.  K is cut into chunks of NG quant groups; the waves of
//    the workgroup take the chunks round-robin.  For its chunk a wave holds the
//    activations in VGPRs (64 bytes per lane, group and batch row) and streams
//    the chunk's codes down the TPW tile-rows, double-buffered: NG contiguous
//    tiles (NG KB at b = 4) per stage, the next stage in flight while one is
//    unpacked.  Activations are thus loaded once per chunk and reused by all
//    16*TPW rows.
//  * Quant params: a chunk's NG scales of one row are one aligned load when
//    NG divides K/128, and its NG zero points always sit in one 32-bit word.
//  * Unpack is exact (dequant.hpp): fp16 (q - z) pairs of consecutive k; the
//    group scale multiplies the group's fp32 partial once per lane (scale and
//    zero are shared by the group -- QFactory review, observation 1).
//  * Reduction: the four k-quarters of a row are summed across lanes with the
//    gfx950 permlane swaps, the waves through LDS in a fixed order, so the
//    result is bitwise deterministic.
#include "common.hpp"
#include "dequant.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

__device__ __forceinline__ h8 cat4(h2 a, h2 b, h2 c, h2 d) {
  return __builtin_bit_cast(h8, u4{as_u32(a), as_u32(b), as_u32(c), as_u32(d)});
}

// Sum of the values held by lanes n, n + 16, n + 32, n + 48 (the four
// k-quarters of tile row n), returned in all four lanes, in the fixed order
// (q0 + q2) + (q1 + q3).
__device__ __forceinline__ float quarter_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t su = __float_as_uint(s);
  const auto b = __builtin_amdgcn_permlane16_swap(su, su, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One lane's codes of one tile: 32 codes = b words, in <= 2 loads.
template <int BITS>
struct LaneCodes {
  uint32_t w[BITS];
  // `off` = lane offset inside the tile (VGPR) or OOB, `soff` = tile offset (SGPR)
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off, uint32_t soff) {
    if constexpr (BITS == 2) {
      const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, CPOL_NT));
      w[0] = v[0];
      w[1] = v[1];
    } else {
#pragma unroll
      for (int h = 0; h < BITS / 4; ++h) {
        const u4 v = bload16<CPOL_NT>(r, off + 1024u * h, soff);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[4 * h + e] = v[e];
      }
    }
  }
};

// Lane byte offset inside a tile (its first word).
template <int BITS>
__device__ __forceinline__ uint32_t lane_off(int lane) {
  return (uint32_t)lane * 4u * (BITS < 4 ? BITS : 4);
}

// NG consecutive fp16 scales of one row in one load (2*NG-byte aligned).
template <int NG>
__device__ __forceinline__ void load_scales(rsrc_t r, uint32_t off, uint32_t soff, uint16_t* s) {
  if constexpr (NG == 1) {
    s[0] = bload2(r, off, soff);
  } else if constexpr (NG == 2) {
    const uint32_t v = bload4(r, off, soff);
    s[0] = (uint16_t)v;
    s[1] = (uint16_t)(v >> 16);
  } else if constexpr (NG == 4) {
    const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = (uint16_t)(v[i / 2] >> (16 * (i % 2)));
  } else {
    static_assert(NG == 8, "NG in {1, 2, 4, 8}");
    const u4 v = bload16(r, off, soff);
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = (uint16_t)(v[i / 2] >> (16 * (i % 2)));
  }
}

// Pipeline variants (groups per chunk NG, ring depth D):
//   V = 0: 64 activation VGPRs per lane (16 per group and batch row), D = 2;
//   V = 1: half the chunk (32 VGPRs), D = 4;
//   V = 2: one group per chunk (16 VGPRs per batch row), D = 4;
//   V = 3: one group per chunk, D = 2.
// Fewer VGPRs buy occupancy (more waves per SIMD to overlap one wave's unpack
// with another's loads); more groups per chunk buy longer contiguous stages.
constexpr int chunk_groups(int bits, bool mfma, int mt, int v) {
  const int base = (bits == 8 ? 2 : 4) / (mfma ? 1 : mt);
  if (v >= 2) return 1;
  return v && base > 1 ? base / 2 : base;
}
constexpr int ring_depth(int v) { return v == 1 || v == 2 ? 4 : 2; }
// Occupancy target (waves per SIMD) the compiler must fit the registers in:
// one-group chunks are sized for 5 (<= 96 VGPRs), the others for 3.
constexpr int waves_per_simd(int ng) { return ng == 1 ? 5 : 3; }

// SAL: K/128 is a multiple of NG, so a chunk's NG scales of one row are one
// aligned load and every chunk is whole.
template <int BITS, bool MFMA, int MT, int NG, int D, int TPW, bool SAL>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(waves_per_simd(NG))))
gemv_tiles_kernel(UniformArgs a) {
  using TR = Uni<BITS>;
  constexpr int PPD = TR::CPD / 2;
  constexpr int ZPW = 32 / BITS;
  constexpr uint32_t ZMASK = (1u << BITS) - 1u;
  constexpr uint32_t TB = 16u * 128u * BITS / 8;  // tile bytes
  constexpr int XR = MFMA ? 1 : MT;               // activation rows per lane
  static_assert(TPW % D == 0, "a chunk's stages fill the ring evenly");
  static_assert(ZPW % NG == 0, "a chunk's zero points share one word");

  // per-wave partials: VALU [WK][TPW][MT][16] floats, MFMA [WK][TPW][64] float4
  extern __shared__ float red[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int WK = blockDim.x >> 6;
  const int n = lane & 15;   // tile row (and, for the MFMA A operand, batch row)
  const int kq = lane >> 4;  // 32-k quarter of the group
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / 128;
  const int NT = (N + 15) / 16;
  const int NC = (G + NG - 1) / NG;
  const int m0 = MFMA ? 0 : blockIdx.y * MT;
  const int rt0 = blockIdx.x * TPW;
  const uint32_t zrow = 4u * ((G * BITS + 31) / 32);
  const uint32_t mg = magic1024x2();
  const uint32_t lw = lane_off<BITS>(lane);

  const rsrc_t rw = make_rsrc(a.wq, (uint32_t)NT * G * TB);
  const rsrc_t rz = make_rsrc(a.zeros, (uint32_t)N * zrow);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * G * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);

  // activation row offsets of this lane (group 0, its k-quarter)
  uint32_t xoff[XR];
#pragma unroll
  for (int r = 0; r < XR; ++r) {
    const int m = MFMA ? n : m0 + r;
    xoff[r] = m < M ? ((uint32_t)m * K + 32u * kq) * 2u : OOB;
  }

  struct St {
    LaneCodes<BITS> c[NG];
    uint16_t s[NG];
    uint32_t z;
  };

  // Every load below is unconditional: a tile-row past the end, a group past
  // K or a chunk past the last one gets an out-of-range offset and reads
  // zeros (scale 0, activation 0), which contributes exactly 0.  Branches
  // here would make the compiler wait for all loads in flight at the join.
  auto load_stage = [&](int t, int c, St& st) {
    const int rt = rt0 + t;
    const int gc0 = c * NG;
    const bool tv = rt < NT;
    const bool cv = gc0 < G;
    const uint32_t row = (uint32_t)rt * 16u + n;  // rows >= N read zeros
    const bool rv = row < (uint32_t)N && cv;
    const uint32_t srow = rv ? row * (uint32_t)G * 2u : OOB;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const bool ok = tv && (SAL ? cv : gc0 + j < G);
      const uint32_t sw = __builtin_amdgcn_readfirstlane(ok ? ((uint32_t)rt * G + gc0 + j) * TB : 0u);
      st.c[j].load(rw, ok ? lw : OOB, sw);
    }
    const uint32_t ss = __builtin_amdgcn_readfirstlane(cv ? 2u * gc0 : 0u);
    if constexpr (SAL) {
      load_scales<NG>(rs, srow, ss, st.s);
    } else {
#pragma unroll
      for (int j = 0; j < NG; ++j) st.s[j] = bload2(rs, gc0 + j < G ? srow : OOB, ss + 2u * j);
    }
    const uint32_t sz = __builtin_amdgcn_readfirstlane(cv ? 4u * (gc0 / ZPW) : 0u);
    st.z = bload4(rz, rv ? row * zrow : OOB, sz);
  };

  u4 xr[NG][XR][4];
  auto load_x = [&](int c) {
    const int gc0 = c * NG;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const bool ok = gc0 + j < G;
      const uint32_t sx = __builtin_amdgcn_readfirstlane(ok ? (uint32_t)(gc0 + j) * 256u : 0u);
#pragma unroll
      for (int r = 0; r < XR; ++r)
#pragma unroll
        for (int v = 0; v < 4; ++v) xr[j][r][v] = bload16(rx, ok ? xoff[r] + 16u * v : OOB, sx);
    }
  };

  float accv[TPW][MT];
  f4 accm[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    accm[t] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < MT; ++m) accv[t][m] = 0.f;
  }

  auto compute = [&](int t, int c, const St& st) {
    const int gc0 = c * NG;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const typename TR::Z zz = TR::zc((st.z >> (BITS * ((gc0 + j) % ZPW))) & ZMASK);
      h2 p[16];  // (q - z) pairs of the lane's 32 consecutive k
#pragma unroll
      for (int d = 0; d < BITS; ++d) TR::deq(st.c[j].w[d], mg, zz, p + d * PPD);
      const float sc = h2f(st.s[j]);
      if constexpr (MFMA) {
        f4 dd = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, xr[j][0][s]),
                                                       cat4(p[4 * s], p[4 * s + 1], p[4 * s + 2], p[4 * s + 3]),
                                                       dd, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) accm[t][i] = fmaf(sc, dd[i], accm[t][i]);
      } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float part = 0.f;
#pragma unroll
          for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int e = 0; e < 4; ++e) part = dot2(p[4 * v + e], as_h2(xr[j][m][v][e]), part);
          accv[t][m] = fmaf(sc, part, accv[t][m]);
        }
      }
    }
  };

  // chunks c = wave, wave + WK, ...; stages (t, c) in order through a ring of
  // D register buffers, D - 1 stages in flight ahead of the one unpacked
  St ring[D];
  int c = wave;
  if (c < NC) {
#pragma unroll
    for (int t = 0; t < D - 1; ++t) load_stage(t, c, ring[t]);
    load_x(c);
  }
  for (; c < NC; c += WK) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int ta = t + D - 1;  // stage to issue (slot of the stage unpacked last)
      if (ta < TPW) {
        load_stage(ta, c, ring[ta % D]);
      } else {
        load_stage(ta - TPW, c + WK, ring[ta % D]);  // next chunk (zeros past the last); same slot
      }
      // keep the schedule as written: unpacking a stage early would hold its
      // expanded pairs in registers and cost occupancy
      __builtin_amdgcn_sched_barrier(0);
      compute(t, c, ring[t % D]);
      __builtin_amdgcn_sched_barrier(0);
    }
    load_x(c + WK);
  }

  if constexpr (MFMA) {
    // lane l holds result rows m = 4 (l / 16) + i of weight row l % 16
    f4* r4 = reinterpret_cast<f4*>(red);
#pragma unroll
    for (int t = 0; t < TPW; ++t) r4[(wave * TPW + t) * 64 + lane] = accm[t];
    __syncthreads();
    for (int e = threadIdx.x; e < TPW * 256; e += blockDim.x) {
      const int r = e & 15, m = (e >> 4) & 15, t = e >> 8;
      const int l = 16 * (m >> 2) + r, i = m & 3;
      float sum = 0.f;
      for (int w = 0; w < WK; ++w) sum += r4[(w * TPW + t) * 64 + l][i];
      const int row = (rt0 + t) * 16 + r;
      if (m < M && row < N) a.y[(size_t)m * N + row] = f2h(sum);
    }
  } else {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float v = quarter_sum(accv[t][m]);
        if (lane < 16) red[((wave * TPW + t) * MT + m) * 16 + lane] = v;
      }
    __syncthreads();
    for (int e = threadIdx.x; e < TPW * MT * 16; e += blockDim.x) {
      const int r = e & 15, m = (e >> 4) % MT, t = (e >> 4) / MT;
      float sum = 0.f;
      for (int w = 0; w < WK; ++w) sum += red[((w * TPW + t) * MT + m) * 16 + r];
      const int row = (rt0 + t) * 16 + r;
      if (m0 + m < M && row < N) a.y[(size_t)(m0 + m) * N + row] = f2h(sum);
    }
  }
}

constexpr size_t LDS_MAX = 64 * 1024;

size_t tiles_lds_bytes(bool mfma, int mt, int tpw, int wk) {
  return mfma ? (size_t)wk * tpw * 64 * 16 : (size_t)wk * tpw * mt * 16 * 4;
}

template <int BITS, bool MFMA, int MT, int V, int TPW>
hipError_t launch_t(const UniformArgs& a, const TileCfg& c, hipStream_t s) {
  constexpr int NG = chunk_groups(BITS, MFMA, MT, V);
  constexpr int D = ring_depth(V);
  if constexpr (TPW % D != 0) {
    return hipErrorInvalidValue;
  } else {
    const int NT = (a.N + 15) / 16;
    const dim3 grid((NT + TPW - 1) / TPW, MFMA ? 1 : (a.M + MT - 1) / MT);
    const dim3 block(64 * c.wk);
    const size_t lds = tiles_lds_bytes(MFMA, MT, TPW, c.wk);
    if (lds > LDS_MAX) return hipErrorInvalidValue;
    if ((a.K / 128) % NG == 0)
      hipLaunchKernelGGL((gemv_tiles_kernel<BITS, MFMA, MT, NG, D, TPW, true>), grid, block, lds, s, a);
    else
      hipLaunchKernelGGL((gemv_tiles_kernel<BITS, MFMA, MT, NG, D, TPW, false>), grid, block, lds, s, a);
    return hipGetLastError();
  }
}

template <int BITS, bool MFMA, int MT, int V>
hipError_t launch_tpw(const UniformArgs& a, const TileCfg& c, hipStream_t s) {
  switch (c.tpw) {
    case 2: return launch_t<BITS, MFMA, MT, V, 2>(a, c, s);
    case 4: return launch_t<BITS, MFMA, MT, V, 4>(a, c, s);
    case 8: return launch_t<BITS, MFMA, MT, V, 8>(a, c, s);
  }
  return hipErrorInvalidValue;
}

template <int BITS, bool MFMA, int MT>
hipError_t launch_v(const UniformArgs& a, const TileCfg& c, hipStream_t s) {
  switch (c.v) {
    case 0: return launch_tpw<BITS, MFMA, MT, 0>(a, c, s);
    case 1: return launch_tpw<BITS, MFMA, MT, 1>(a, c, s);
    case 2: return launch_tpw<BITS, MFMA, MT, 2>(a, c, s);
    case 3: return launch_tpw<BITS, MFMA, MT, 3>(a, c, s);
  }
  return hipErrorInvalidValue;
}

template <int BITS>
hipError_t launch_b(const UniformArgs& a, const TileCfg& c, hipStream_t s) {
  if (c.mfma) return launch_v<BITS, true, 1>(a, c, s);
  switch (c.mt) {
    case 1: return launch_v<BITS, false, 1>(a, c, s);
    case 2: return launch_v<BITS, false, 2>(a, c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

TileCfg pick_tiles(int bits, int M, int N, int K, bool mfma) {
  TileCfg c;
  c.mfma = mfma;
  c.mt = mfma || M <= 1 ? 1 : 2;
  c.v = 0;
  const int ng = chunk_groups(bits, mfma, c.mt, c.v);
  const int G = K / 128;
  const int nc = (G + ng - 1) / ng;
  const long nt = (N + 15) / 16;
  const long mtiles = mfma ? 1 : (M + c.mt - 1) / c.mt;
  // every chunk in flight at once (up to 8 waves), then as many tile-rows
  // per workgroup as still leave >= 4096 waves
  c.wk = nc < 8 ? nc : 8;
  c.tpw = 8;
  while (c.tpw > 2 && ((nt + c.tpw - 1) / c.tpw) * mtiles * c.wk < 4096) c.tpw /= 2;
  while (c.tpw > 2 && tiles_lds_bytes(mfma, c.mt, c.tpw, c.wk) > LDS_MAX) c.tpw /= 2;
  return c;
}

hipError_t launch_gemv_tiles(const UniformArgs& a, const TileCfg& c, hipStream_t s) {
  if (c.wk < 1 || c.wk > 8) return hipErrorInvalidValue;
  switch (a.bits) {
    case 2: return launch_b<2>(a, c, s);
    case 4: return launch_b<4>(a, c, s);
    case 8: return launch_b<8>(a, c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
