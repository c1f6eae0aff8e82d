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
#include <cstdlib>
#include <type_traits>

#include "common.hpp"
#include "dequant.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

__device__ __forceinline__ h8 cat4(h2 a, h2 b, h2 c, h2 d) {
  return __builtin_bit_cast(h8, u4{as_u32(a), as_u32(b), as_u32(c), as_u32(d)});
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
//   V = 3: one group per chunk, D = 2;
//   V = 4, 5: one group per chunk, one tile-row per workgroup, D = 4 / 8
//   chunks in flight (VALU engine with staged activations only): a small
//   layer gives each wave only a few chunks, and all of them are issued at
//   once instead of one memory round trip per chunk.
// Fewer VGPRs buy occupancy (more waves per SIMD to overlap one wave's unpack
// with another's loads); more groups per chunk buy longer contiguous stages.
constexpr int chunk_groups(int bits, bool mfma, int mt, int v) {
  const int base = (bits == 8 ? 2 : 4) / (mfma ? 1 : mt);
  if (v >= 2) return 1;
  return v && base > 1 ? base / 2 : base;
}
constexpr int ring_depth(int v) { return v == 5 ? 8 : (v == 1 || v == 2 || v == 4 ? 4 : 2); }
// Occupancy target (waves per SIMD) the compiler must fit the registers in:
// one-group chunks are sized for 5 (<= 96 VGPRs), the others for 3.
constexpr int waves_per_simd(int ng) { return ng == 1 ? 5 : 3; }
// Workgroup size bound: one-group chunks fit 16 waves (<= 128 VGPRs each).
constexpr int max_threads(int ng) { return ng == 1 ? 1024 : 512; }

// SAL: K/128 is a multiple of NG, so a chunk's NG scales of one row are one
// aligned load and every chunk is whole.
// XLDS: the workgroup stages its activation rows in LDS once (VALU: its MT
// rows; MFMA: all M rows) and every lane reads its 64-byte slice of a group
// from there.  The sixteen lanes of a k-quarter share that slice (VALU), so
// loading it per lane through the vector memory path would request 16x the
// bytes it uses.  MFMA lanes of batch rows past M read row M - 1 instead of
// zeros: those rows of the product are never stored.
// SP: also add the Tile-COO fp16 outliers of the workgroup's rows (outlier
// variant): see sparse_compute below.
// PLDS: the workgroup's 16 TPW rows of scales and of packed zero points are
// two contiguous blocks; they are staged in LDS with coalesced 16-byte loads,
// so a chunk costs one weight load per lane and tile instead of three
// (per-lane scale and zero loads touch 16 rows' cache lines for every 1 KB
// of codes).
// XD (MFMA, activations too large to stage whole, one-group chunks of
// several tile-rows): each wave streams its chunks' activation blocks (the
// batch rows x 128 k) through a two-slot LDS ring with 16-byte loads straight
// into LDS, a chunk ahead.  Such a load covers 4 rows x 256 contiguous bytes
// (8 cache lines); the per-lane A-fragment loads it replaces touch 32 lines
// each.  A chunk's A fragments and quant params are read from LDS before the
// next chunk's load is issued, so the wait for a slot's load is never a
// wait for the one behind it.
// FULL (one tile-row of one-group chunks, either engine):
// K/128 is a multiple of the ring depth times the waves (a round of the
// two-stage loop is two chunks per wave), so every chunk a wave unpacks
// inside its loop lies inside K and the selects for chunks past the last
// (activation pad, zero point, scale) drop out; the loads issued ahead past
// the last chunk still read zeros.
template <int BITS, bool MFMA, int MT, int NG, int D, int TPW, bool SAL, bool XLDS, bool SP, bool PLDS,
          bool XD = false, bool FULL = false>
__global__ void __launch_bounds__(max_threads(NG)) __attribute__((amdgpu_waves_per_eu(waves_per_simd(NG))))
gemv_tiles_kernel(UniformArgs a) {
  using TR = Uni<BITS>;
  constexpr int PPD = TR::CPD / 2;
  constexpr int ZPW = 32 / BITS;
  constexpr uint32_t ZMASK = (1u << BITS) - 1u;
  constexpr uint32_t TB = 16u * 128u * BITS / 8;  // tile bytes
  constexpr int XR = MFMA ? 1 : MT;               // activation rows per lane
  // DEEP: one tile-row and a ring of D > 2 one-group chunks
  constexpr bool DEEP = TPW == 1 && D > 2;
  static_assert(TPW % D == 0 || (TPW == 1 && D == 2) || DEEP, "a chunk's stages fill the ring evenly");
  static_assert(!DEEP || (XLDS && NG == 1), "the deep chunk ring keeps no activations in registers");
  static_assert(ZPW % NG == 0, "a chunk's zero points share one word");
  static_assert(!XD || (MFMA && !XLDS && !SP && NG == 1 && TPW >= D), "the activation ring: MFMA, one-group chunks");
  static_assert(!FULL || (TPW == 1 && NG == 1), "whole chunk rounds: one tile-row of one-group chunks");

  // LDS: [staged activations: XM x K halves, XLDS only] [staged scales and
  // zero points of the TPW tile-rows, PLDS only] then the per-wave partials: VALU
  // [WK][TPW][MT][16] floats, MFMA [WK][TPW][64] float4
  extern __shared__ __attribute__((aligned(16))) float smem[];
  // Z2T (2-bit codes, kernels that pass the staging barrier before their
  // loop): the five zero-point constants of each z in 0..3, built once per
  // workgroup (32 bytes per z), so a group reads them instead of building
  // them from its zero point (a multiply-add and five shift-ors per group)
  constexpr bool Z2T = BITS == 2 && (XLDS || PLDS || SP);
  __shared__ __attribute__((aligned(16))) uint32_t z2tab[Z2T ? 32 : 4];
  if constexpr (Z2T) {
    if (threadIdx.x < 4) {
      const typename TR::Z zt = TR::zc(threadIdx.x);
#pragma unroll
      for (int k = 0; k < 5; ++k) z2tab[8 * threadIdx.x + k] = as_u32(zt.c[k]);
    }
  }

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
  // the deep rings select a chunk past the last by its descriptor (an empty
  // one: every load reads zeros), a scalar select, instead of by a vector
  // select of the lane offset per chunk
  const rsrc_t rw0 = make_rsrc(a.wq, 0u);
  const rsrc_t rz = make_rsrc(a.zeros, (uint32_t)N * zrow);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * G * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);
  // staged activation row stride in halves: K, then a zero pad that groups
  // past K read instead (they add s = 0 times a finite value)
  const int XK = K + 32;
  const int XM = MFMA ? min(M, 16) : MT;  // staged activation rows
  // XD: the activation ring first (per wave two slots of XMR rows x 256
  // bytes, XMR = the batch rows rounded up to 4), which the partials reuse
  // after the loop
  const int XMR = (min(M, 16) + 3) & ~3;
  const uint32_t xslot = 256u * XMR;
  const size_t ringb = !XD ? 0
                      : (size_t)WK * 2 * xslot > (size_t)WK * TPW * 64 * 16 ? (size_t)WK * 2 * xslot
                                                                            : (size_t)WK * TPW * 64 * 16;
  char* const pbase = reinterpret_cast<char*>(smem) + (XLDS ? (size_t)XM * XK * 2 : ringb);
  const uint32_t psb = PLDS ? (32u * TPW * G + 15u) & ~15u : 0u;  // 16 TPW rows x G scales, 16-byte padded
  const uint32_t pzb = PLDS ? 16u * TPW * zrow : 0u;                // 16 TPW rows of packed zero points
  const uint16_t* ps = reinterpret_cast<const uint16_t*>(pbase);
  const uint32_t* pz = reinterpret_cast<const uint32_t*>(pbase + psb);
  float* red = XD ? smem : reinterpret_cast<float*>(pbase + psb + pzb);
  const u4* xs = reinterpret_cast<const u4*>(smem);

  // outlier variant (SP): LDS after the partials (see sparse_lds_bytes), per
  // wave: VPB 64-record batches loaded straight into LDS, a batch's row keys
  // [64] and its products [PR][64] (VALU: the MT batch rows; MFMA: the M
  // batch rows rounded up to 4, at most PM = 16); after the waves' slots, the
  // workgroup's tile pointers [TPW G + 1]
  constexpr int VPB = 4;
  constexpr int PM = MFMA ? 16 : MT;
  const int PR = MFMA ? min((M + 3) & ~3, 16) : MT;
  const int SPW = 256 * VPB + 256 + PR * 256;  // bytes per wave
  uint32_t* vrec = nullptr;  // [VPB][64] prefetched records
  uint32_t* vrow = nullptr;  // [64] row keys of a batch
  float* vprod = nullptr;    // [PM][64] products of a batch
  uint32_t* vptr = nullptr;  // the workgroup's tile pointers
  if constexpr (SP) {
    const size_t redb = MFMA ? (size_t)WK * TPW * 64 * 16 : (size_t)WK * TPW * MT * 16 * 4;
    char* b = reinterpret_cast<char*>(red) + redb + (size_t)wave * SPW;
    vrec = reinterpret_cast<uint32_t*>(b);
    vrow = reinterpret_cast<uint32_t*>(b + 256 * VPB);
    vprod = reinterpret_cast<float*>(b + 256 * VPB + 256);
    vptr = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(red) + redb + (size_t)WK * SPW);
  }

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
      if constexpr (DEEP)
        st.c[j].load(ok ? rw : rw0, lw, sw);
      else
        st.c[j].load(rw, ok ? lw : OOB, sw);
    }
    if constexpr (PLDS) return;  // quant params come from LDS
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

  // activation buffers: one, or two when a single tile-row per workgroup
  // leaves nothing else to overlap the next chunk's activation loads with
  constexpr int XB = TPW < D ? 2 : 1;
  u4 xr[XLDS ? 1 : XB][XLDS ? 1 : NG][XR][4];
  auto load_x = [&](int c, int b) {
    if constexpr (XLDS || XD) return;
    const int gc0 = c * NG;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const bool ok = gc0 + j < G;
      const uint32_t sx = __builtin_amdgcn_readfirstlane(ok ? (uint32_t)(gc0 + j) * 256u : 0u);
#pragma unroll
      for (int r = 0; r < XR; ++r)
#pragma unroll
        for (int v = 0; v < 4; ++v) xr[XLDS ? 0 : b][XLDS ? 0 : j][r][v] = bload16(rx, ok ? xoff[r] + 16u * v : OOB, sx);
    }
  };

  // XD: the current chunk's quant params, read from LDS with its A fragments
  uint16_t xd_s[XD && PLDS ? TPW : 1];
  uint32_t xd_z[XD && PLDS ? TPW : 1];
  // XD: activation block of chunk c (group c) into ring slot `slot`: load j
  // covers rows 4 j .. 4 j + 3, lane l writing piece l % 16 of row
  // 4 j + l / 16, which holds k-piece (l % 16) ^ row (the swizzle keeps the
  // 16 rows of an A-fragment read on distinct banks); rows past M and chunks
  // past the last read zeros
  // (offsets formed at issue: kept in registers across the loop they would
  // cost occupancy)
  auto xd_issue = [&](int c, int slot) {
    if constexpr (XD) {
      const uint32_t so = __builtin_amdgcn_readfirstlane(c < G ? 256u * (uint32_t)c : 0u);
      char* dst = reinterpret_cast<char*>(smem) + (size_t)(wave * 2 + slot) * xslot;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 4 * j + kq;
        if (4 * j < XMR)  // (wave-uniform)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rx, (__attribute__((address_space(3))) void*)(dst + 1024 * j), 16,
              row < M && c < G ? ((uint32_t)row * K + 8u * (uint32_t)(n ^ row)) * 2u : OOB, so, 0, 0);
      }
    }
  };
  // XD: the A fragments of the chunk in `slot` (batch row n, or row XMR - 1
  // for n >= XMR: those result rows are never stored) into the activation
  // registers, and its quant params (read once per chunk: read per tile-row
  // from LDS instead, they measured up to 20% slower)
  auto xd_read = [&](int c, int slot) {
    if constexpr (XD) {
      const int row = min(n, XMR - 1);
      const u4* xb = reinterpret_cast<const u4*>(reinterpret_cast<const char*>(smem) +
                                                 (size_t)(wave * 2 + slot) * xslot + 256u * row);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) xr[0][0][0][s4] = xb[(4 * kq + s4) ^ row];
      if constexpr (PLDS) {
        const bool gin = c < G;
        const int g = min(c, G - 1);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const uint16_t sv = ps[(16 * t + n) * G + g];
          const uint32_t zv = pz[(16 * t + n) * (int)(zrow / 4) + g / ZPW];
          xd_s[t] = gin ? sv : (uint16_t)0;
          xd_z[t] = gin ? zv : 0u;
        }
      }
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

  auto compute = [&](int t, int c, const St& st, int b) {
    const int gc0 = c * NG;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      uint32_t zw = st.z;
      uint16_t sj = st.s[j];
      if constexpr (PLDS) {  // (a chunk past the last: scale 0, zero point 0)
        if constexpr (XD) {
          sj = xd_s[t];
          zw = xd_z[t];
        } else {
          // unconditional reads at a clamped group, then a select: a read
          // under a condition would become a branch inside the pipelined loop
          // (the several-tile-row loop, XB = 1, computes only chunks below
          // NC, and whole ones when SAL: no select there, as for xin)
          const bool gin = FULL || (SAL && XB == 1) || gc0 + j < G;
          const int g = min(gc0 + j, G - 1);
          const uint16_t sv = ps[(16 * t + n) * G + g];
          const uint32_t zv = pz[(16 * t + n) * (int)(zrow / 4) + g / ZPW];
          sj = gin ? sv : (uint16_t)0;
          zw = gin ? zv : 0u;
        }
      }
      const float sc = h2f(sj);
      const uint32_t zq = (zw >> (BITS * ((gc0 + j) % ZPW))) & ZMASK;
      const typename TR::Z zz = [&] {
        if constexpr (Z2T) {
          typename TR::Z r;
          const u4 e = *reinterpret_cast<const u4*>(&z2tab[8 * zq]);
#pragma unroll
          for (int k = 0; k < 4; ++k) r.c[k] = as_h2(e[k]);
          r.c[4] = as_h2(z2tab[8 * zq + 4]);
          return r;
        } else {
          return TR::zc(zq);
        }
      }();
      h2 p[16];  // (q - z) pairs of the lane's 32 consecutive k
#pragma unroll
      for (int d = 0; d < BITS; ++d) TR::deq(st.c[j].w[d], mg, zz, p + d * PPD);
      if constexpr (MFMA) {
        f4 dd = f4{0.f, 0.f, 0.f, 0.f};
        // A operand: batch row n (row XM - 1 for n >= XM), the lane's k slice
        const bool xin = FULL || (SAL && XB == 1) || gc0 + j < G;
        const int xa = (min(n, XM - 1) * XK + (xin ? 128 * (gc0 + j) + 32 * kq : K)) / 8;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, XLDS ? xs[xa + s] : xr[b][j][0][s]),
                                                       cat4(p[4 * s], p[4 * s + 1], p[4 * s + 2], p[4 * s + 3]),
                                                       dd, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) accm[t][i] = fmaf(sc, dd[i], accm[t][i]);
      } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float part = 0.f;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            // x[m0 + m][128 (gc0 + j) + 32 kq + 8 v .. + 8], or the zero pad
            const bool xin = FULL || (SAL && XB == 1) || gc0 + j < G;
            // (unsigned: every term is non-negative, so the division is a shift)
            const u4 xv = XLDS ? xs[((uint32_t)(m * XK) + (xin ? 128u * (uint32_t)(gc0 + j) + 32u * kq : (uint32_t)K)) / 8u + v]
                               : xr[b][j][m][v];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              part = v == 0 && e == 0 ? dot2_first(p[0], as_h2(xv[0])) : dot2(p[4 * v + e], as_h2(xv[e]), part);
          }
          accv[t][m] = fmaf(sc, part, accv[t][m]);
        }
      }
    }
  };

  // chunks c = wave, wave + WK, ...; stages (t, c) in order through a ring of
  // D register buffers, D - 1 stages in flight ahead of the one unpacked.
  // The scheduling barriers keep the schedule as written: unpacking a stage
  // early would hold its expanded pairs in registers and cost occupancy.
  St ring[D];
  int c = wave;
  // Activations of rows m0 .. m0 + MT - 1 into LDS, 16 distinct bytes per
  // lane and load; rows >= M read zeros.  Four loads in flight per lane.
  // (row stride XK; the 4 pad vectors of each row get zeros: their loads are
  // out of range.)  The first pass is issued before the weight prefetch and
  // written after it, so waiting for the activations never waits for the
  // weights behind them (loads complete in order); the barrier waits for LDS
  // traffic only, leaving the weight stages in flight.
  const int X8 = XK / 8, n16 = XM * X8;
  const float x8inv = 1.0f / (float)X8;
  auto x_pass = [&](int i0, u4* v) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * blockDim.x;
      // row of vector i (VALU: MT rows, known here; i >= n16 loads nothing)
      const int m = MFMA ? div_small(i, X8, x8inv) : (MT == 1 ? 0 : (i >= X8 ? 1 : 0));
      const int k8 = i - m * X8;
      v[u] = bload16(rx, i < n16 && m0 + m < M && k8 < K / 8 ? ((uint32_t)(m0 + m) * K + 8u * k8) * 2u : OOB);
    }
  };
  u4 xfirst[XLDS ? 4 : 1];
  // quant params of the TPW tile-rows: scale vectors [0, psb / 16), then
  // zero point vectors; rows past N read zeros
  const int np16 = (int)((psb + pzb) / 16);
  auto p_pass = [&](int i) -> u4 {
    const uint32_t sv = psb / 16u;
    return (uint32_t)i < sv ? bload16(rs, (uint32_t)rt0 * 32u * G + 16u * i)
                            : bload16(rz, i < np16 ? (uint32_t)rt0 * 16u * zrow + 16u * (i - sv) : OOB);
  };
  u4 pfirst;
  // Outlier variant: the tile pointers of the workgroup's tile-rows (nvt
  // tiles, nvt + 1 entries), thread i loading entries i, i + blockDim, ...
  // (at most SPP per thread here; more in stage_x)
  const rsrc_t rtp = make_rsrc(a.tile_ptr, ((uint32_t)NT * G + 1u) * 4u);
  constexpr int SPP = 2;
  const int nvt = (min(TPW, NT - rt0)) * G;
  uint32_t pv[SPP];
  auto stage_x_issue = [&]() {
    if constexpr (XLDS) x_pass(threadIdx.x, xfirst);
    if constexpr (PLDS) pfirst = p_pass(threadIdx.x);
    if constexpr (SP) {
#pragma unroll
      for (int u = 0; u < SPP; ++u) {
        const int i = threadIdx.x + u * blockDim.x;
        pv[u] = bload4(rtp, i <= nvt ? ((uint32_t)rt0 * G + i) * 4u : OOB);
      }
    }
  };
  auto stage_x = [&]() {
    if constexpr (XLDS) {
      u4* xw = reinterpret_cast<u4*>(smem);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (threadIdx.x + u * blockDim.x < n16) xw[threadIdx.x + u * blockDim.x] = xfirst[u];
      for (int i0 = threadIdx.x + 4 * blockDim.x; i0 < n16; i0 += 4 * blockDim.x) {
        u4 v[4];
        x_pass(i0, v);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (i0 + u * blockDim.x < n16) xw[i0 + u * blockDim.x] = v[u];
      }
    }
    if constexpr (PLDS) {
      u4* pw = reinterpret_cast<u4*>(pbase);
      if ((int)threadIdx.x < np16) pw[threadIdx.x] = pfirst;
      for (int i = threadIdx.x + blockDim.x; i < np16; i += blockDim.x) pw[i] = p_pass(i);
    }
    if constexpr (SP) {
#pragma unroll
      for (int u = 0; u < SPP; ++u) {
        const int i = threadIdx.x + u * blockDim.x;
        if (i <= nvt) vptr[i] = pv[u];
      }
      for (int i = threadIdx.x + SPP * blockDim.x; i <= nvt; i += blockDim.x)
        vptr[i] = bload4(rtp, ((uint32_t)rt0 * G + i) * 4u);
    }
    lds_barrier();
  };
  // Outliers (FlashQuant abstract: an fp16 sparse path fused with the
  // low-bit dense one, sharing activations and outputs; Tile-COO records).
  // A Tile-COO tile is the 16 x 128 tile of the dense layout, so the records
  // of a workgroup's tile-rows are one contiguous range [vbeg, vend).  The
  // tile pointers are staged with the activations; right after the staging
  // barrier each wave's first VPB 64-record batches (batches w, w + WK, ...)
  // go straight into LDS, issued behind the first weight stages, and arrive
  // during the dense loop.  After the loop each wave walks its batches
  // (sparse_batch) and adds the sums of its lanes' records into its dense
  // partials, which the fixed-order reduction then adds like any other
  // partial.  Every product is exact and the order of the sums is fixed, so
  // the result is deterministic.  Record fields are masked into the
  // tile-row and a tile's count is bounded, so malformed records stay in
  // bounds.
  const rsrc_t rrec = make_rsrc(a.tile_rec, (uint32_t)a.nnz * 4u);
  uint32_t vbeg = 0, vend = 0;
  auto sparse_issue = [&]() {
    if constexpr (SP) {
      vbeg = __builtin_amdgcn_readfirstlane(vptr[0]);
      vend = __builtin_amdgcn_readfirstlane(vptr[nvt]);
      // (a tile holds at most 2048 records: malformed pointers stay bounded)
      vend = vend < vbeg ? vbeg : min(vend, vbeg + 2048u * (uint32_t)nvt);
#pragma unroll
      for (int i = 0; i < VPB; ++i) {
        const uint32_t r = vbeg + 64u * (wave + WK * i) + lane;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rrec, vrec + 64 * i, 4, r < vend ? r * 4u : OOB, 0, 0, 0);
      }
    }
  };
  // Lanes of a wave exchange data through its LDS slot; LDS operations of
  // one wave complete in order, but without a fence the compiler may assume no
  // other lane wrote what this lane reads (and forward its own earlier store).
  auto wave_fence = [] { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); };
  // A batch of 64 records.  Lane i takes record i: its tile is the last one
  // whose range starts at or before it (binary search over the staged
  // pointers); its products v x[m][k] (exact) for the batch rows and its row
  // key (tile-row t, row r) = 16 t + r go to the wave's slot.  Lane (r,
  // quarter p) then adds, in record order, the products of the batch's
  // quarter p whose row is r, for every batch row (VALU: its MT rows; MFMA:
  // the rows m < M, four at a time).  The quarters are added in a fixed order
  // at the end (VALU: by the reduction; MFMA: one quarter sum per row, added
  // by the lanes that hold that row of the matrix-core result).
  const _Float16* xh = reinterpret_cast<const _Float16*>(smem);
  constexpr int SR = MFMA ? 16 : MT;  // batch rows a lane sums
  float sacc[TPW][SR];
  auto sparse_batch = [&](uint32_t rec, uint32_t idx) {
    const bool ok = idx < vend;
    int j = 0;
    for (int st = 1 << (31 - __builtin_clz(nvt)); st > 0; st >>= 1)
      if (j + st < nvt && vptr[j + st] <= idx) j += st;
    const int t = TPW == 1 ? 0 : (j >= G ? 1 : 0);
    const uint32_t col = 128u * (uint32_t)(j - t * G) + (rec & 127u);
    const float v = h2f((uint16_t)(rec >> 16));
#pragma unroll
    for (int m = 0; m < PM; ++m) {
      if (m < PR) {  // (wave-uniform: the rows of the slot)
        const int xm = MFMA ? m : m0 + m;  // batch row (rows past M add nothing)
        float xv = 0.f;
        if (xm < M) {
          if constexpr (XLDS) xv = (float)xh[m * XK + col];  // (staged rows: the batch rows from m0)
          else xv = h2f(bload2(rx, ok ? ((uint32_t)xm * K + col) * 2u : OOB));
        }
        vprod[m * 64 + lane] = ok ? v * xv : 0.f;
      }
    }
    vrow[lane] = ok ? ((rec >> 8) & 15u) + 16u * t : 0xFFFFu;
    wave_fence();  // (other lanes read these)
    // the quarter's 16 keys, and its products four rows at a time, read with
    // 16-byte reads that every lane of the quarter shares, then added
    // branch-free where the row matches
    u4 kv[4];
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) kv[v4] = reinterpret_cast<const u4*>(vrow)[4 * kq + v4];
#pragma unroll
    for (int g4 = 0; g4 < SR; g4 += 4) {
      constexpr int RG = SR < 4 ? SR : 4;
      if (g4 < PR) {  // (wave-uniform)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {  // four records at a time
          u4 pv[RG];
#pragma unroll
          for (int i = 0; i < RG; ++i) pv[i] = reinterpret_cast<const u4*>(vprod + (g4 + i) * 64)[4 * kq + v4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t key = kv[v4][e];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
              const bool hit = key == (uint32_t)(n + 16 * tt);
#pragma unroll
              for (int i = 0; i < RG; ++i) sacc[tt][g4 + i] += hit ? __uint_as_float(pv[i][e]) : 0.f;
            }
          }
        }
      }
    }
    wave_fence();  // (the slot is rewritten by the next batch)
  };
  // A wave's first batch runs early in the dense loop, right after the
  // first chunk's next stage loads are issued: the batches (in LDS) were the
  // last loads before those, so an exact vmcnt waits for them and no more,
  // and the batch is worked through while the weight stages are in flight
  // (run after the loop, its latency adds to every workgroup's).  Its other
  // batches, and a wave's with no chunk, still run after the loop: more
  // sparse work inside the loop would hold back the weight stream.  Only the
  // VALU engine at one batch row with at most three stages in flight does
  // so: with the matrix core's 16 row sums per lane, or a fourth stage's
  // registers, the sums held across the loop no longer fit the register
  // budget and spill.
  constexpr bool SP_EARLY = SP && !MFMA && MT == 1 && D <= 3;
  int sp_i = 0;  // the wave's next batch (wave-uniform)
  auto sparse_zero = [&]() {
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
      for (int i = 0; i < SR; ++i) sacc[t][i] = 0.f;
  };
  // in a loop's first chunk, after N vector memory instructions issued
  // behind the batch loads
  auto sparse_early = [&](auto n) {
    if constexpr (SP_EARLY) {
      constexpr int N = decltype(n)::value;
      static_assert(N < 64, "vmcnt range");
      if (sp_i == 0) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));  // vmcnt(N)
        sparse_zero();
        const uint32_t b0 = vbeg + 64u * wave;
        if (b0 < vend) sparse_batch(vrec[lane], b0 + lane);
        sp_i = 1;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto sparse_compute = [&]() {
    if constexpr (SP) {
      if (sp_i == 0) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the batches are in LDS (issued long before)
        sparse_zero();
      }
      // (after an early batch the others are in LDS too: their loads came
      // before the ones the early wait covered)
      for (int i = sp_i;; ++i) {  // wave-uniform
        const uint32_t b0 = vbeg + 64u * (wave + WK * i);
        if (b0 >= vend) break;
        const uint32_t idx = b0 + lane;
        const uint32_t rec = i < VPB ? vrec[64 * i + lane] : bload4(rrec, idx < vend ? idx * 4u : OOB);
        sparse_batch(rec, idx);
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int i = 0; i < SR; ++i) {
          if constexpr (MFMA) {
            // lane (r, p) holds result rows 4 p .. 4 p + 3 of weight row r
            if (i < M) {  // (wave-uniform)
              const float sm = quarter_sum(sacc[t][i]);
              accm[t][i & 3] += kq == (i >> 2) ? sm : 0.f;
            }
          } else {
            accv[t][i] += sacc[t][i];
          }
        }
    }
  };

  // vector memory instructions of one load_stage, and of one load_x
  constexpr int SLD = NG * (BITS == 8 ? 2 : 1) + (PLDS ? 0 : (SAL ? 1 : NG) + 1);
  constexpr int XLD = XLDS || XD ? 0 : NG * XR * 4;
  stage_x_issue();
  // (a wave with no chunk at all, c >= NC, reads zeros: no branch here)
  if constexpr (XB == 1) {
#pragma unroll
    for (int t = 0; t < D - 1; ++t) load_stage(t, c, ring[t]);
    load_x(c, 0);
    xd_issue(c, 0);
    if constexpr (XLDS || PLDS || SP) stage_x();
    sparse_issue();
    int xsl = 0;  // XD: ring slot of chunk c
    // XD: the compiler does not order reads of a ring slot after the loads
    // into it, so the waits are explicit.  Before the loop: everything (the
    // first slot, the first stages).  At the top of each chunk: its slot's
    // loads, which the previous chunk's TPW weight stages followed (loads
    // complete in order; the scheduling barriers keep the issue order).  The
    // next chunk's loads go into the other slot, read (into registers) a
    // chunk ago.
    constexpr int XLPS = (BITS == 8 ? 2 : 1) + (PLDS ? 0 : 2);  // vector memory instructions per stage
    constexpr int XW = TPW * XLPS;
    static_assert(XW < 64, "vmcnt range");
    constexpr int XVMW = (XW & 15) | (0x7 << 4) | (0xF << 8) | ((XW >> 4) << 14);  // s_waitcnt vmcnt(XW)
    if constexpr (XD) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    for (; c < NC; c += WK) {
      if constexpr (XD) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(XVMW);
        xd_read(c, xsl);
        __builtin_amdgcn_sched_barrier(0);
        xd_issue(c + WK, xsl ^ 1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int ta = t + D - 1;  // stage to issue (slot of the stage unpacked last)
        if (ta < TPW) {
          load_stage(ta, c, ring[ta % D]);
        } else {
          load_stage(ta - TPW, c + WK, ring[ta % D]);  // next chunk (zeros past the last); same slot
        }
        if (t == 0) sparse_early(std::integral_constant<int, SLD>{});
        __builtin_amdgcn_sched_barrier(0);
        compute(t, c, ring[t % D], 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      load_x(c + WK, 0);
      xsl ^= 1;
    }
  } else if constexpr (DEEP) {
    // one tile-row, D chunks in flight: chunk c + i WK sits in slot i % D
    // (chunks past the last read zeros and add nothing)
#pragma unroll
    for (int i = 0; i < D - 1; ++i) load_stage(0, c + i * WK, ring[i]);
    stage_x();
    sparse_issue();
    for (; c < NC; c += D * WK) {
#pragma unroll
      for (int i = 0; i < D; ++i) {
        load_stage(0, c + (i + D - 1) * WK, ring[(i + D - 1) % D]);
        if (i == 0) sparse_early(std::integral_constant<int, SLD>{});
        __builtin_amdgcn_sched_barrier(0);
        compute(0, c + i * WK, ring[i], 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    // one tile-row, two stages: chunks alternate between slot/buffer 0 and 1
    // (a chunk past the last reads zeros and adds nothing)
    load_stage(0, c, ring[0]);
    load_x(c, 0);
    if constexpr (XLDS || PLDS || SP) stage_x();
    sparse_issue();
    for (; c < NC; c += 2 * WK) {
      load_stage(0, c + WK, ring[1]);
      load_x(c + WK, 1);
      sparse_early(std::integral_constant<int, SLD + XLD>{});
      __builtin_amdgcn_sched_barrier(0);
      compute(0, c, ring[0], 0);
      __builtin_amdgcn_sched_barrier(0);
      load_stage(0, c + 2 * WK, ring[0]);
      load_x(c + 2 * WK, 0);
      __builtin_amdgcn_sched_barrier(0);
      compute(0, c + WK, ring[1], 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  sparse_compute();

  if constexpr (MFMA) {
    if constexpr (XD) {
      // the partials reuse the activation ring: every load into it has
      // landed and every wave is past its last read
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      __syncthreads();
    }
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
    reduce_waves(red, TPW * MT * 16, WK, [&](int e, float sum) {
      const int r = e & 15, m = (e >> 4) % MT, t = (e >> 4) / MT;
      const int row = (rt0 + t) * 16 + r;
      if (m0 + m < M && row < N) a.y[(size_t)(m0 + m) * N + row] = f2h(sum);
    });
  }
}

constexpr size_t LDS_MAX = 64 * 1024;

size_t tiles_lds_bytes(bool mfma, int mt, int tpw, int wk) {
  return mfma ? (size_t)wk * tpw * 64 * 16 : (size_t)wk * tpw * mt * 16 * 4;
}
// activation staging: MT rows (VALU) or all M rows (MFMA) of K + 32 halves
constexpr size_t XLDS_MAX = 64 * 1024 + 128;
size_t xlds_bytes(bool mfma, int mt, int M, int K) { return (size_t)(mfma ? (M < 16 ? M : 16) : mt) * (K + 32) * 2; }

// LDS of the outlier variant beyond the dense kernel's: per wave four
// 64-record batches, a batch's row keys and its products (MT batch rows, or
// on the MFMA engine the M rows rounded up to 4), then the workgroup's
// tpw G + 1 tile pointers
size_t sparse_lds_bytes(bool mfma, int mt, int wk, int tpw, int K, int M) {
  const int pr = mfma ? (((M + 3) & ~3) < 16 ? ((M + 3) & ~3) : 16) : mt;
  return (size_t)wk * (256 * 4 + 256 + 256 * pr) + ((size_t)tpw * (K / 128) + 1) * 4;
}

constexpr size_t LDS_ALL = 160 * 1024;  // gfx950 LDS per workgroup
// static LDS of the kernel beside its dynamic share (the 2-bit zero-point
// constant table, Z2T): counted in both limits below
constexpr size_t z2t_lds(int bits) { return bits == 2 ? 128 : 0; }

template <int BITS, bool MFMA, int MT, int NG, int D, int TPW, bool SAL, bool XLDS, bool SP, bool PLDS,
          bool XD = false, bool FULL = false>
hipError_t launch_k(const UniformArgs& a, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
  auto kern = &gemv_tiles_kernel<BITS, MFMA, MT, NG, D, TPW, SAL, XLDS, SP, PLDS, XD, FULL>;
  if (lds + z2t_lds(BITS) > 64 * 1024) {
    static bool raised = false;  // one-time opt-in above the default dynamic LDS limit
    if (!raised) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)(LDS_ALL - z2t_lds(BITS)));
      if (e != hipSuccess) return e;
      raised = true;
    }
  }
  hipLaunchKernelGGL(kern, grid, block, lds, s, a);
  return hipGetLastError();
}

// staged quant params of tpw tile-rows (PLDS): 16 tpw rows of G fp16 scales,
// 16-byte padded, then 16 tpw rows of packed zero points
size_t params_lds_bytes(int bits, int K, int tpw) {
  const size_t G = K / 128;
  return (32 * tpw * G + 15) / 16 * 16 + 16 * tpw * 4 * ((G * bits + 31) / 32);
}

template <int BITS, bool MFMA, int MT, int NG, int D, int TPW, bool XL, bool SP>
hipError_t launch_p(const UniformArgs& a, bool sal, bool plds, bool xd, dim3 grid, dim3 block, size_t lds,
                    hipStream_t s, bool full = false) {
  // the activation ring (XD): the matrix-core engine with activations not
  // staged whole, one-group chunks of several tile-rows, no outliers
  constexpr bool XD_OK = MFMA && !XL && !SP && NG == 1 && TPW >= D && TPW >= 2 && TPW <= 4 && !(BITS == 8 && TPW == 4);
  if constexpr (XD_OK) {
    if (xd) {
      if (!sal) return hipErrorInvalidValue;
      return plds ? launch_k<BITS, MFMA, MT, NG, D, TPW, true, XL, SP, true, true>(a, grid, block, lds, s)
                  : launch_k<BITS, MFMA, MT, NG, D, TPW, true, XL, SP, false, true>(a, grid, block, lds, s);
    }
  }
  if (xd) return hipErrorInvalidValue;
  if constexpr (TPW == 1 && NG == 1) {
    // one-group chunks: a group's scale is always one whole, aligned load
    if (!sal) return hipErrorInvalidValue;
    {
      if (full)
        return plds ? launch_k<BITS, MFMA, MT, NG, D, TPW, true, XL, SP, true, false, true>(a, grid, block, lds, s)
                    : launch_k<BITS, MFMA, MT, NG, D, TPW, true, XL, SP, false, false, true>(a, grid, block, lds, s);
    }
    return plds ? launch_k<BITS, MFMA, MT, NG, D, TPW, true, XL, SP, true>(a, grid, block, lds, s)
                : launch_k<BITS, MFMA, MT, NG, D, TPW, true, XL, SP, false>(a, grid, block, lds, s);
  } else {
    // Staged quant params with several tile-rows: on the matrix-core engine
    // (sweeps of the 8B and 70B layers: 6-17% faster at M = 4..16; on the
    // VALU engine at M = 1 its several-group chunks already take one scale
    // load per tile, and staging measured up to 20% slower), and where the
    // kernel still fits its registers (8 tile-rows of one-group chunks or of
    // 2-bit codes spill).
    constexpr bool PLDS_OK = MFMA && !(TPW == 8 && (NG == 1 || BITS == 2));
    if constexpr (PLDS_OK)
      if (sal && plds) return launch_k<BITS, MFMA, MT, NG, D, TPW, true, XL, SP, true>(a, grid, block, lds, s);
    return sal ? launch_k<BITS, MFMA, MT, NG, D, TPW, true, XL, SP, false>(a, grid, block, lds, s)
               : launch_k<BITS, MFMA, MT, NG, D, TPW, false, XL, SP, false>(a, grid, block, lds, s);
  }
}

template <int BITS, bool MFMA, int MT, int V, int TPW, bool SP = false>
hipError_t launch_t(const UniformArgs& a, const TileCfg& c, hipStream_t s) {
  constexpr int NG = chunk_groups(BITS, MFMA, MT, V);
  constexpr int D = ring_depth(V);
  constexpr bool DEEP = TPW == 1 && D > 2;
  if constexpr (TPW % D != 0 && !(TPW == 1 && D == 2 && NG == 1) && !(DEEP && !MFMA && NG == 1)) {
    return hipErrorInvalidValue;
  } else {
    const int NT = (a.N + 15) / 16;
    const dim3 grid((NT + TPW - 1) / TPW, MFMA ? 1 : (a.M + MT - 1) / MT);
    const dim3 block(64 * c.wk);
    const size_t red = tiles_lds_bytes(MFMA, MT, TPW, c.wk);
    if (red > LDS_MAX || 64 * c.wk > max_threads(NG)) return hipErrorInvalidValue;
    const size_t xl = xlds_bytes(MFMA, MT, a.M, a.K);
    size_t xmax = XLDS_MAX;
    if (const char* e = tune_env("QGEMV_XLDS_MAX")) xmax = (size_t)std::atol(e);  // tuning override (bytes)
    const bool xlds = xl <= xmax;
    // (the buffer bounds check drops a 16-byte load that straddles the end of
    // an array, so both arrays must end on a 16-byte boundary: N % 8 == 0 does)
    const size_t G = a.K / 128, zbytes = (size_t)a.N * 4 * ((G * BITS + 31) / 32);
    bool plds = reinterpret_cast<uintptr_t>(a.scales) % 16 == 0 && reinterpret_cast<uintptr_t>(a.zeros) % 16 == 0 &&
                (size_t)a.N * G * 2 % 16 == 0 && zbytes % 16 == 0;
    if (const char* e = tune_env("QGEMV_PLDS")) plds = plds && e[0] == '1';  // tuning override
    // chunk scales in one load: whole chunks and a 2*NG-byte aligned base
    const bool sal = (a.K / 128) % NG == 0 && reinterpret_cast<uintptr_t>(a.scales) % (2 * NG) == 0;
    // the activation ring (matrix cores, activations not staged whole): per
    // wave two slots of the batch rows (rounded up to 4) x 256 bytes, which
    // the partials reuse after the loop
    // (the wider variants would spill).  Used where the launch shape asks for
    // it (pick_tiles: where it measured faster).
    bool xd = MFMA && !xlds && !SP && NG == 1 && TPW >= D && TPW >= 2 && TPW <= 4 && !(BITS == 8 && TPW == 4) && sal;
    bool xd_want = c.xd;
    if (const char* e = tune_env("QGEMV_XDMA")) xd_want = e[0] == '2' || (e[0] == '1' && xd_want);  // tuning override
    xd = xd && xd_want;
    const size_t ring = (size_t)c.wk * 2 * 256 * ((std::min(a.M, 16) + 3) & ~3);
    const size_t rest = xd ? std::max(ring, red)
                           : (xlds ? xl : 0) + red + (SP ? sparse_lds_bytes(MFMA, MT, c.wk, TPW, a.K, a.M) : 0);
    const size_t lds_all = LDS_ALL - z2t_lds(BITS);
    if (rest + params_lds_bytes(BITS, a.K, TPW) > lds_all) plds = false;  // (long K: stage nothing)
    const size_t lds = rest + (plds ? params_lds_bytes(BITS, a.K, TPW) : 0);
    if (lds > lds_all) return hipErrorInvalidValue;
    if constexpr (DEEP) {
      if (!xlds) return hipErrorInvalidValue;  // the deep ring reads activations from LDS only
      // every wave's chunks fill whole rounds of the ring
      const int nc = (int)(a.K / 128 + NG - 1) / NG;
      bool full = nc % (D * c.wk) == 0;
      if (const char* e = tune_env("QGEMV_FULL_ROUNDS")) full = full && e[0] == '1';  // tuning override
      return launch_p<BITS, MFMA, MT, NG, D, TPW, true, SP>(a, sal, plds, false, grid, block, lds, s, full);
    } else {
      if (xlds) {
        // one tile-row, two stages: whole rounds as for the deep rings
        const int nc = (int)(a.K / 128 + NG - 1) / NG;
        bool full = TPW == 1 && nc % (D * c.wk) == 0;
        if (const char* e = tune_env("QGEMV_FULL_ROUNDS")) full = full && e[0] == '1';  // tuning override
        return launch_p<BITS, MFMA, MT, NG, D, TPW, true, SP>(a, sal, plds, false, grid, block, lds, s, full);
      }
      return launch_p<BITS, MFMA, MT, NG, D, TPW, false, SP>(a, sal, plds, xd, grid, block, lds, s);
    }
  }
}

template <int BITS, bool MFMA, int MT, int V>
hipError_t launch_tpw(const UniformArgs& a, const TileCfg& c, hipStream_t s) {
  switch (c.tpw) {
    case 1:
      // (the 8-deep ring holds 8-bit stages only by spilling)
      if constexpr (V == 3 || ((V == 4 || (V == 5 && BITS < 8)) && !MFMA)) return launch_t<BITS, MFMA, MT, V, 1>(a, c, s);
      return hipErrorInvalidValue;
  }
  if constexpr (V >= 4) {
    return hipErrorInvalidValue;  // the deep rings exist for one tile-row only
  } else {
    switch (c.tpw) {
      case 2: return launch_t<BITS, MFMA, MT, V, 2>(a, c, s);
      case 4: return launch_t<BITS, MFMA, MT, V, 4>(a, c, s);
      case 8: return launch_t<BITS, MFMA, MT, V, 8>(a, c, s);
    }
    return hipErrorInvalidValue;
  }
}

template <int BITS, bool MFMA, int MT>
hipError_t launch_v(const UniformArgs& a, const TileCfg& c, hipStream_t s) {
  switch (c.v) {
    case 0: return launch_tpw<BITS, MFMA, MT, 0>(a, c, s);
    case 1: return launch_tpw<BITS, MFMA, MT, 1>(a, c, s);
    case 2: return launch_tpw<BITS, MFMA, MT, 2>(a, c, s);
    case 3: return launch_tpw<BITS, MFMA, MT, 3>(a, c, s);
    case 4: return launch_tpw<BITS, MFMA, MT, 4>(a, c, s);
    case 5: return launch_tpw<BITS, MFMA, MT, 5>(a, c, s);
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

// Launch shape per engine and layer shape, fitted to full sweeps on MI355X
// over the Llama-3-8B / 70B decode layers (cache-cold weights, W2/W4/W8,
// M = 1..16; within 2-3% of the per-shape best in total):
//  * VALU (batch 1): one tile-row per workgroup with staged quant params and
//    one-group chunks -- 16 waves for long K, 4 when the grid is already wide,
//    a 4-deep chunk ring for the shortest K -- except the widest layers and
//    4-bit layers of 384-512 tile-rows, which take two tile-rows and
//    four-group chunks;
//  * MFMA (batch >= 2), 2- and 4-bit codes: one tile-row for narrow layers
//    (at most 256 tile-rows; 16 waves at M = 5..7 for K < 12288; two
//    tile-rows for long K from M = 12); otherwise 2 or 4 tile-rows of
//    one-group chunks with staged quant params (16 waves up to M = 6, for
//    K >= 8192 and from M = 12, where the activation ring frees the
//    registers the wide workgroups need; else 8), two tile-rows with the
//    ring for the widest layers at M = 5..8, and 8 tile-rows with half
//    chunks for the widest 4-bit layers at M >= 9.  8-bit codes keep the
//    earlier fit (several-group chunks).
//  * The activation ring (matrix cores, activations not staged whole) for
//    K >= 16384, from M = 12, and for the shapes that set it above.
TileCfg pick_tiles(int bits, int M, int N, int K, bool mfma) {
  TileCfg c;
  c.mfma = mfma;
  c.mt = mfma || M <= 1 ? 1 : 2;
  const int G = K / 128;
  const long nt = (N + 15) / 16;
  auto set = [&](int tpw, int wk, int v) {
    c.tpw = tpw;
    c.wk = wk;
    c.v = v;
  };
  if (!mfma) {
    if (nt >= 2048 || (bits == 4 && G <= 32 && nt > 256 && nt <= 512)) {
      set(2, 8, 0);
    } else {
      const int wk = G >= 96 ? 16 : (nt >= 1024 ? 4 : 8);
      set(1, wk, wk <= 8 && (nt <= 256 || nt >= 1024) ? 4 : 3);
    }
  } else if (nt <= 256) {  // narrow layers: one tile-row per workgroup
    if (M <= 2) set(1, 16, 3);
    else if (M <= 4) set(1, G >= 96 ? 8 : 16, 3);
    else if (M >= 12 && G >= 96 && bits != 8) set(2, 16, 3);  // (long K: two tile-rows, the activation ring)
    else if (M <= 7 && G < 96 && bits != 8) set(1, 16, 3);
    else set(1, M <= 8 ? 8 : 4, 3);
  } else if (bits == 8) {
    if (M >= 8 && nt >= 1536) {
      if (M >= 9) set(8, 8, 0);
      else set(4, 4, 0);
    } else if (M <= 2) {
      if (nt >= 2048 || G >= 128) set(2, 8, 0);
      else set(1, nt >= 1024 ? 4 : 8, 3);
    } else if (M <= 4) {
      if (nt >= 1536) set(4, nt >= 2048 ? 4 : 8, 0);
      else if (G >= 128) set(2, 8, 0);
      else set(1, 8, 3);
    } else {
      if (nt >= 1536) set(4, 4, 0);
      else if (nt >= 640) set(4, 8, 0);
      else set(2, M <= 8 ? 8 : 4, 0);
    }
  } else if (M <= 2) {
    if (nt >= 2048 || G >= 128) set(2, 16, 3);
    else if (bits == 2 && nt >= 1024) set(2, 8, 3);
    else set(1, nt >= 1024 ? 4 : 8, 3);
  } else if (M <= 4) {
    if (nt >= 2048) set(bits == 4 ? 2 : 4, 8, 3);
    else if (nt >= 1024) set(4, 8, 3);
    else if (nt >= 640 && G < 128) set(4, 16, 3);
    else set(2, 16, 3);
  } else {
    if (nt >= 1536) {
      if (bits == 4 && M >= 9) set(8, nt >= 2048 ? 4 : 8, 1);  // half chunks keep 8 tile-rows of stages in registers
      else if (M <= 8 && nt >= 2048) set(2, 4, 3), c.xd = true;
      else set(4, 8, 3);
    } else if (nt >= 640 && G < 128) {
      set(4, 16, 3);
    } else if (M <= 8 && G >= 64) {
      set(2, 16, 3), c.xd = true;
    } else {
      set(2, G >= 128 || M >= 12 || M <= 6 ? 16 : 8, 3);
    }
  }
  // the activation ring (where the shape and the activations allow it):
  // long K, or from M = 12, or as set above
  if (mfma && (G >= 128 || M >= 12)) c.xd = true;
  // never more waves than chunks of groups
  const int ng = chunk_groups(bits, mfma, c.mt, c.v);
  const int nc = (G + ng - 1) / ng;
  if (c.wk > nc) c.wk = nc < 1 ? 1 : nc;
  return c;
}

// Outlier variant.  VALU (sweeps of the 8B and 70B layers at M = 1): one
// tile-row of one-group chunks -- 16 waves for long K, 4 on wide layers,
// else 8, with the 4-deep ring on layers of at most 256 tile-rows and the
// 2-deep one elsewhere -- except from 2048 tile-rows on, where two tile-rows
// with four-group chunks and 4 waves win.  MFMA: the uniform W4 shapes,
// restricted to one tile-row with the 2-deep ring and two tile-rows with
// four-group chunks.
TileCfg pick_outlier(int M, int N, int K, bool mfma) {
  TileCfg c = pick_tiles(4, M, N, K, mfma);
  if (!mfma) {
    const long nt = (N + 15) / 16;
    const int G = K / 128;
    if (nt >= 2048) {
      c.tpw = 2;
      c.v = 0;
      c.wk = 4;
      const int nc = (G + chunk_groups(4, false, c.mt, 0) - 1) / chunk_groups(4, false, c.mt, 0);
      if (c.wk > nc) c.wk = nc;
    } else {
      c.tpw = 1;
      c.wk = G >= 96 ? 16 : (nt >= 1024 ? 4 : 8);
      c.v = nt <= 256 && c.wk <= 8 ? 4 : 3;
      if (c.wk > G) c.wk = G;
    }
  } else if (c.tpw == 1) {
    c.v = 3;
  } else {
    c.tpw = 2;
    c.v = 0;
    if (c.wk > 8) c.wk = 8;  // (several-group chunks: at most 512 threads)
    const int nc = (K / 128 + chunk_groups(4, mfma, c.mt, 0) - 1) / chunk_groups(4, mfma, c.mt, 0);
    if (c.wk > nc) c.wk = nc;
  }
  // halve the waves until the launch's LDS fits (staged activations and
  // quant params, partials, the sparse phase's slots): long K with batch
  // rows staged leaves less room for per-wave scratch
  size_t xl = xlds_bytes(mfma, c.mt, M, K);
  if (xl > XLDS_MAX) xl = 0;
  const size_t fixed = xl + params_lds_bytes(4, K, c.tpw);
  while (c.wk > 1 && fixed + tiles_lds_bytes(mfma, c.mt, c.tpw, c.wk) +
                             sparse_lds_bytes(mfma, c.mt, c.wk, c.tpw, K, M) > LDS_ALL)
    c.wk = (c.wk + 1) / 2;
  return c;
}

hipError_t launch_gemv_outlier(const UniformArgs& a, const TileCfg& c, hipStream_t s) {
  if (a.bits != 4 || c.wk < 1 || c.wk > 16) return hipErrorInvalidValue;
  const int key = c.tpw * 10 + c.v;
  if (c.mfma) {
    if (key == 13) return launch_t<4, true, 1, 3, 1, true>(a, c, s);
    if (key == 20) return launch_t<4, true, 1, 0, 2, true>(a, c, s);
  } else if (c.mt == 1) {
    if (key == 13) return launch_t<4, false, 1, 3, 1, true>(a, c, s);
    if (key == 14) return launch_t<4, false, 1, 4, 1, true>(a, c, s);
    if (key == 20) return launch_t<4, false, 1, 0, 2, true>(a, c, s);
  } else if (c.mt == 2) {
    if (key == 13) return launch_t<4, false, 2, 3, 1, true>(a, c, s);
    if (key == 14) return launch_t<4, false, 2, 4, 1, true>(a, c, s);
    if (key == 20) return launch_t<4, false, 2, 0, 2, true>(a, c, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_tiles(const UniformArgs& a, const TileCfg& c, hipStream_t s) {
  if (c.wk < 1 || c.wk > 16) return hipErrorInvalidValue;
  switch (a.bits) {
    case 2: return launch_b<2>(a, c, s);
    case 4: return launch_b<4>(a, c, s);
    case 8: return launch_b<8>(a, c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
