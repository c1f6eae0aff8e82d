// Fused LUT-dequantize-and-multiply for 4-bit codes with a 16-entry fp16
// lookup table (NF4-style) and a per-64-block fp16 scale, at decode batch
// M <= 16, on gfx950:
//
//   y[m, n] = sum_k x[m, k] * LUT[q[n, k]] * a[n, k/64]
//
// The Fast NF4 Dequantization Kernels page: the 16-level table lives on chip
// (shared memory, 64 bytes per block) instead of being re-read per element,
// with simplified indexing; the 64-weight block scale is applied per block.
//
// Design (gfx950):
//  * Codes use the same tiled device layout as the uniform W4 kernels (one
//    16-row x 128-k tile per quant group, lane l = row l % 16, k-quarter
//    l / 16), so the packer and the streaming are shared.  A lane's 32 k lie in
//    one 64-block, so the block scale is one per lane and group.
//  * Lookup: an LDS pair table holds, for every code byte b, the fp16 pair
//    (LUT[b & 15], LUT[b >> 4]), replicated 64 times lane-major: entry b of copy
//    c at byte (64 b + c) * 4.  Lane l always reads copy l, so every lookup is
//    bank-conflict-free, and its address (b << 8) | (4 l) is one v_perm_b32 of
//    the code word and 4 l.  One LDS read yields two dequantized weights.
//  * In the device field order byte j of a code word holds the k offsets
//    (0,2), (4,6), (1,3), (5,7) for j = 0..3.  The activations are staged in
//    LDS with each 8-k run stored in that order, so a table pair meets its
//    activation pair as loaded: per 8 weights, 4 v_perm + 4 ds_read_b32 +
//    4 v_dot2 (one VALU instruction per weight).
//  * Persistent workgroups: the 64 KB table allows two workgroups per CU (of
//    up to 16 waves at one batch row), and building it costs as much as
//    streaming a few tile-rows, so the grid holds only the resident
//    workgroups; each builds its table and stages the
//    activations once, then walks row groups, issuing the next group's first
//    chunks before reducing the current one (the barriers wait for LDS only).
//  * Streaming, pipeline, work split and reduction follow the uniform kernel:
//    branch-free non-temporal tile loads through a D-slot register ring,
//    permlane quarter sums, LDS wave sums in fixed order (deterministic).
//  * Block scales: per lane with its codes, or (one batch row, workgroups
//    that walk several row groups) staged in LDS a row group ahead with
//    coalesced loads.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

constexpr int TABLE_COPIES = 64;
constexpr uint32_t TABLE_BYTES = 256u * TABLE_COPIES * 4u;  // 64 KB

// activation area: MT staged rows, and at least 1 KB (it first holds the 256
// pair values the table copies are made from)
__host__ __device__ constexpr size_t xarea_bytes(int mt, int K) {
  return (size_t)mt * (K + 32) * 2 > 1024 ? (size_t)mt * (K + 32) * 2 : 1024;
}

// Block scales of NG consecutive groups of one row: the lane's 64-block is
// (2 g + kq / 2); one aligned load when SAL.
template <int NG>
__device__ __forceinline__ void load_block_scales(rsrc_t r, uint32_t rowoff, uint32_t soff, int half,
                                                  uint16_t* s) {
  if constexpr (NG == 1) {
    const uint32_t v = bload4(r, rowoff, soff);
    s[0] = (uint16_t)(v >> (16 * half));
  } else if constexpr (NG == 2) {
    const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, rowoff, soff, 0));
    s[0] = (uint16_t)(v[0] >> (16 * half));
    s[1] = (uint16_t)(v[1] >> (16 * half));
  } else {
    static_assert(NG == 4, "NG in {1, 2, 4}");
    const u4 v = bload16(r, rowoff, soff);
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = (uint16_t)(v[j] >> (16 * half));
  }
}

// TPW tile-rows per workgroup (1, 2), NG groups per chunk, MT activation
// rows per workgroup; with one tile-row, D chunks per wave in a ring (D - 1
// loads ahead).  SAL: K/128 is a multiple of NG and the block scales are
// 4*NG-byte aligned, so a chunk's scales are one load.
// BS (one tile-row, one-group chunks): a row group's block scales (16 rows
// x K/64, one contiguous block of the [N, K/64] array) are staged in LDS
// with coalesced 4-byte loads (at most two per thread), issued a whole row
// group ahead; per-lane scale loads would touch 16 rows' cache lines for
// every 1 KB tile of codes.
template <int MT, int NG, int TPW, int D, bool SAL, bool BS>
__global__ void __launch_bounds__(MT == 1 ? 1024 : 512, MT == 1 ? 4 : 2) gemv_lut4_kernel(Lut4Args a) {
  static_assert(!BS || (SAL && NG == 1 && TPW == 1), "staged block scales: one tile-row, one-group chunks");
  // LDS: the pair table (64 KB, static: its address is a compile-time
  // constant, so a lookup's address is the v_perm result itself, with no add
  // of a dynamic base), then dynamic [activations MT x XK halves, 8-k runs
  // permuted (xarea_bytes)][partials][BS: two buffers of 16 rows x SW words
  // of block-scale pairs]
  __shared__ __attribute__((aligned(16))) uint32_t ltab[TABLE_BYTES / 4];
  extern __shared__ __attribute__((aligned(16))) uint32_t lsm[];
  char* const lds = reinterpret_cast<char*>(lsm);
  const char* const tab = reinterpret_cast<const char*>(ltab);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int WK = blockDim.x >> 6;
  const int n = lane & 15;
  const int kq = lane >> 4;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / 128;
  const int KB = K / 64;  // block scales per row
  const int NT = (N + 15) / 16;
  const int NC = (G + NG - 1) / NG;
  const int m0 = blockIdx.y * MT;
  const int NRG = (NT + TPW - 1) / TPW;  // row groups (TPW tile-rows each)
  int rt0 = blockIdx.x * TPW;             // the current row group's first tile-row
  const int XK = K + 32;  // staged row stride (halves): K, then a zero pad
  const uint32_t lane4 = 4u * lane;
  float* const red = reinterpret_cast<float*>(lds + xarea_bytes(MT, K));
  // staged block scales (BS): word g of row r holds the scales of group g
  // (64-blocks 2g, 2g + 1); SW is odd, so the 16 rows of one read fall on
  // distinct banks
  const int SW = G | 1;
  uint32_t* const sbuf = reinterpret_cast<uint32_t*>(lds + xarea_bytes(MT, K) + (size_t)WK * TPW * MT * 64);

  const rsrc_t rw = make_rsrc(a.wq, (uint32_t)NT * G * 1024u);
  const rsrc_t ra = make_rsrc(a.absmax, (uint32_t)N * KB * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);
  const rsrc_t rl = make_rsrc(a.lut, 32u);

  struct St {
    u4 c[NG];
    uint16_t s[NG];
  };

  // all loads unconditional: out-of-range tile-rows, groups and chunks read
  // zeros (scale 0), so they add exactly 0
  auto load_stage = [&](int t, int c, St& st) {
    const int rt = rt0 + t;
    const int gc0 = c * NG;
    const bool tv = rt < NT;
    const bool cv = gc0 < G;
    const uint32_t row = (uint32_t)rt * 16u + n;
    const bool rv = row < (uint32_t)N && cv;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const bool ok = tv && (SAL ? cv : gc0 + j < G);
      const uint32_t sw = __builtin_amdgcn_readfirstlane(ok ? ((uint32_t)rt * G + gc0 + j) * 1024u : 0u);
      st.c[j] = bload16<CPOL_NT>(rw, ok ? 16u * lane : OOB, sw);
    }
    if constexpr (BS) return;  // block scales come from LDS
    const uint32_t ss = __builtin_amdgcn_readfirstlane(cv ? 4u * gc0 : 0u);
    if constexpr (SAL) {
      load_block_scales<NG>(ra, rv ? row * (uint32_t)KB * 2u : OOB, ss, kq >> 1, st.s);
    } else {
#pragma unroll
      for (int j = 0; j < NG; ++j)
        st.s[j] = bload2(ra, rv && gc0 + j < G ? (row * (uint32_t)KB + (kq >> 1)) * 2u : OOB, ss + 4u * j);
    }
  };

  float acc[TPW][MT];

  // With several tile-rows per workgroup a chunk's activation slices are read
  // from LDS once into registers and reused for every tile-row; with one they
  // are read per use.
  constexpr bool XREG = TPW >= 2;
  u4 xc[XREG ? NG : 1][XREG ? MT : 1][4];
  auto xslice = [&](int c, int j, int m, int d) -> u4 {
    const int gc0 = c * NG;
    const bool xin = (SAL && TPW >= 2) || gc0 + j < G;
    const uint32_t xk = xin ? 128u * (gc0 + j) + 32u * kq : (uint32_t)K;
    return *reinterpret_cast<const u4*>(lds + ((uint32_t)m * XK + xk + 8u * d) * 2u);
  };
  auto load_xc = [&](int c) {
    if constexpr (XREG) {
#pragma unroll
      for (int j = 0; j < NG; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int d = 0; d < 4; ++d) xc[j][m][d] = xslice(c, j, m, d);
    }
  };

  int sb = 0;  // the staged block-scale buffer of the current row group (BS)
  auto compute = [&](int t, int c, const St& st) {
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      float part[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) part[m] = 0.f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        u4 xv[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) xv[m] = XREG ? xc[XREG ? j : 0][XREG ? m : 0][d] : xslice(c, j, m, d);
        const uint32_t w = st.c[j][d];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          // (code byte jb << 8) | 4 lane: entry jb of this lane's table copy
          const uint32_t addr = __builtin_amdgcn_perm(w, lane4, 0x0C0C0000u | ((4u + jb) << 8));
          const h2 pr = as_h2(*reinterpret_cast<const uint32_t*>(tab + addr));
#pragma unroll
          for (int m = 0; m < MT; ++m) part[m] = dot2(pr, as_h2(xv[m][jb]), part[m]);
        }
      }
      float sc;
      if constexpr (BS) {
        // the lane's 64-block of group c: half kq / 2 of word c of row n
        const uint32_t wv = sbuf[(sb * 16 + n) * SW + c];
        sc = h2f((uint16_t)(wv >> (16 * (kq >> 1))));
      } else {
        sc = h2f(st.s[j]);
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[t][m] = fmaf(sc, part[m], acc[t][m]);
    }
  };

  constexpr int R = TPW >= 2 ? 2 : D;
  St ring[R];
  // the first chunks of row group rt0 (zeros past the last chunk or row)
  auto prologue = [&]() {
    if constexpr (TPW >= 2) {
      load_stage(0, wave, ring[0]);
    } else {
#pragma unroll
      for (int k = 0; k + 1 < R; ++k) load_stage(0, wave + k * WK, ring[k]);
    }
  };
  // BS: words i = threadIdx.x + e blockDim.x (e < 2) of tile-row rt's block
  // scales (16 G words; tile-rows past the last and rows past N read zeros),
  // and their stores into buffer b (row i / G, word i % G)
  // (the second word only where the workgroup has fewer threads than words:
  // a uniform branch; the LDS word offsets are the same for every row group)
  using BSv = uint32_t[2];
  const bool bs2 = BS && (int)blockDim.x < 16 * G;
  int bsoff[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = threadIdx.x + e * (int)blockDim.x;
    const int r = i / G;
    bsoff[e] = BS && i < 16 * G ? r * SW + (i - r * G) : -1;
  }
  auto bs_issue = [&](int rt, BSv& v) {
    if constexpr (BS) {
      const uint32_t so = __builtin_amdgcn_readfirstlane(rt < NT ? (uint32_t)rt * 64u * (uint32_t)G : 0u);
      v[0] = bload4(ra, rt < NT && bsoff[0] >= 0 ? 4u * threadIdx.x : OOB, so);
      if (bs2) v[1] = bload4(ra, rt < NT && bsoff[1] >= 0 ? 4u * (threadIdx.x + blockDim.x) : OOB, so);
    }
  };
  auto bs_store = [&](int b, const BSv& v) {
    if constexpr (BS) {
      if (bsoff[0] >= 0) sbuf[b * 16 * SW + bsoff[0]] = v[0];
      if (bs2 && bsoff[1] >= 0) sbuf[b * 16 * SW + bsoff[1]] = v[1];
    }
  };
  // Start-up loads, in the order they are needed: the table entries, then the
  // first pass of activations, then the weight prefetch.  A wave's loads
  // return in order, so building the table waits for the 32-byte table only,
  // and staging the activations never waits for the weights behind them.
  uint32_t tlo[4], thi[4];  // table values of entries e = threadIdx.x + j blockDim.x
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = threadIdx.x + j * (int)blockDim.x;
    tlo[j] = bload2(rl, e < 256 ? 2u * (e & 15) : OOB);
    thi[j] = bload2(rl, e < 256 ? 2u * (e >> 4) : OOB);
  }
  const int X8 = XK / 8, n16 = MT * X8;
  auto x_pass = [&](int i0, u4* v) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * blockDim.x;
      // row of vector i (MT rows; i >= n16 loads nothing)
      const int m = MT == 1 ? 0 : (i >= X8 ? 1 : 0);
      const int k8 = i - m * X8;
      v[u] = bload16(rx, i < n16 && m0 + m < M && k8 < K / 8 ? ((uint32_t)(m0 + m) * K + 8u * k8) * 2u : OOB);
    }
  };
  u4 xfirst[4];
  x_pass(threadIdx.x, xfirst);
  BSv bsfirst;
  bs_issue(rt0, bsfirst);
  prologue();  // weights in flight while the tables fill

  // pair table: 256 pair values, then 64 lane-major copies of each
  {
    uint32_t* pairs = reinterpret_cast<uint32_t*>(lds);  // scratch in the x area
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = threadIdx.x + j * (int)blockDim.x;
      if (e < 256) pairs[e] = tlo[j] | (thi[j] << 16);
    }
    lds_barrier();
    // 16 bytes (four copies of one pair) per write: piece i holds copies
    // 4 (i % 16) .. + 3 of entry i / 16
    constexpr int PIECES = 256 * TABLE_COPIES / 4;
    for (int i = threadIdx.x; i < PIECES; i += blockDim.x) {
      const uint32_t v = pairs[i / (TABLE_COPIES / 4)];
      reinterpret_cast<u4*>(ltab)[i] = u4{v, v, v, v};
    }
    lds_barrier();  // (LDS only: the weight prefetch stays in flight)
  }
  // activations of rows m0 .. m0 + MT - 1; each 8-k run stored as
  // (x0,x2),(x4,x6),(x1,x3),(x5,x7); the 4 pad runs per row read zeros
  {
    u4* xw = reinterpret_cast<u4*>(lds);
    auto put = [&](int i0, const u4* v) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const u4 p = {__builtin_amdgcn_perm(v[u][1], v[u][0], 0x05040100u),
                      __builtin_amdgcn_perm(v[u][3], v[u][2], 0x05040100u),
                      __builtin_amdgcn_perm(v[u][1], v[u][0], 0x07060302u),
                      __builtin_amdgcn_perm(v[u][3], v[u][2], 0x07060302u)};
        if (i0 + u * blockDim.x < n16) xw[i0 + u * blockDim.x] = p;
      }
    };
    put(threadIdx.x, xfirst);
    for (int i0 = threadIdx.x + 4 * blockDim.x; i0 < n16; i0 += 4 * blockDim.x) {
      u4 v[4];
      x_pass(i0, v);
      put(i0, v);
    }
    bs_store(0, bsfirst);
    lds_barrier();
  }

  // Persistent: the table and the staged activations serve every row group
  // rg = blockIdx.x, blockIdx.x + gridDim.x, ...  The next group's first
  // chunks are issued before this group's reduction.
  for (int rg = blockIdx.x; rg < NRG; rg += gridDim.x) {
  BSv bsnext;
  bs_issue((rg + (int)gridDim.x) * TPW, bsnext);  // the next row group's block scales
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[t][m] = 0.f;
  int c = wave;
  if constexpr (TPW >= 2) {
    for (; c < NC; c += WK) {
      load_xc(c);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        if (t + 1 < TPW)
          load_stage(t + 1, c, ring[(t + 1) & 1]);
        else
          load_stage(0, c + WK, ring[(t + 1) & 1]);  // next chunk (zeros past the last)
        __builtin_amdgcn_sched_barrier(0);
        compute(t, c, ring[t & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else {
    // one tile-row: chunks c = wave + i WK through the R-slot ring; the loads
    // stay unconditional (zeros past the last chunk), only the compute is
    // skipped there
    for (; c < NC; c += R * WK) {
#pragma unroll
      for (int k = 0; k < R; ++k) {
        load_stage(0, c + (k + R - 1) * WK, ring[(k + R - 1) % R]);
        __builtin_amdgcn_sched_barrier(0);
        if (c + k * WK < NC) compute(0, c + k * WK, ring[k]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  const int rtc = rt0;
  rt0 = (rg + (int)gridDim.x) * TPW;
  prologue();  // past the last group: rows out of range, zeros

#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v = quarter_sum(acc[t][m]);
      if (lane < 16) red[((wave * TPW + t) * MT + m) * 16 + lane] = v;
    }
  bs_store(sb ^ 1, bsnext);  // (its last reader was the group before this one)
  lds_barrier();  // LDS only: the next group's loads stay in flight
  reduce_waves(red, TPW * MT * 16, WK, [&](int e, float sum) {
    const int r = e & 15, m = (e >> 4) % MT, t = (e >> 4) / MT;
    const int row = (rtc + t) * 16 + r;
    if (m0 + m < M && row < N) a.y[(size_t)(m0 + m) * N + row] = f2h(sum);
  });
  lds_barrier();  // the partial area is written again by the next group
  sb ^= 1;
  }
}

constexpr size_t LUT4_LDS_LIMIT = 160 * 1024;

size_t lut4_lds_bytes(int mt, int tpw, int wk, int K) {
  return TABLE_BYTES + xarea_bytes(mt, K) + (size_t)wk * tpw * mt * 16 * 4;
}

// staged block scales (BS): two buffers of 16 rows x (G | 1) words
size_t lut4_bs_bytes(int K) { return 2u * 16u * 4u * (size_t)((K / 128) | 1); }

// kernel per scale mode: 0 per-group scale loads, 1 one aligned load per
// chunk (SAL), 2 staged block scales (BS)
template <int MT, int NG, int TPW, int D>
const void* lut4_kernel(int mode) {
  if constexpr (NG == 1 && TPW == 1)
    if (mode == 2) return reinterpret_cast<const void*>(&gemv_lut4_kernel<MT, NG, TPW, D, true, true>);
  return mode ? reinterpret_cast<const void*>(&gemv_lut4_kernel<MT, NG, TPW, D, true, false>)
              : reinterpret_cast<const void*>(&gemv_lut4_kernel<MT, NG, TPW, D, false, false>);
}

template <int MT, int NG, int TPW, int D>
hipError_t launch_l(const Lut4Args& a, const Lut4Cfg& c, hipStream_t s) {
  const int NT = (a.N + 15) / 16;
  const int NRG = (NT + TPW - 1) / TPW;
  const int MY = (a.M + MT - 1) / MT;
  const int G = a.K / 128;
  const dim3 block(64 * c.wk);
  const size_t total = lut4_lds_bytes(MT, TPW, c.wk, a.K);
  if (total > LUT4_LDS_LIMIT) return hipErrorInvalidValue;
  const bool sal = G % NG == 0 && reinterpret_cast<uintptr_t>(a.absmax) % (4 * NG) == 0;
  static bool raised = false;  // one-time opt-in to the whole LDS beside the static table
  if (!raised) {
    const int dmax = (int)(LUT4_LDS_LIMIT - TABLE_BYTES);
    for (int m = 0; m < 3; ++m) {
      const hipError_t e = hipFuncSetAttribute(lut4_kernel<MT, NG, TPW, D>(m), hipFuncAttributeMaxDynamicSharedMemorySize, dmax);
      if (e != hipSuccess) return e;
    }
    raised = true;
  }
  // persistent grid: no more workgroups than are resident at once (each
  // builds its table once and walks row groups).  Residency per CU is asked
  // once per (scale mode, waves, LDS size) and remembered.
  static int occ[3][17];
  static size_t occ_lds[3][17];
  int dev = 0, cus = 0;
  hipError_t e0 = hipGetDevice(&dev);
  if (e0 == hipSuccess) e0 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e0 != hipSuccess) return e0;
  auto slots_of = [&](int mode, size_t lds, long& slots) -> hipError_t {
    if (occ_lds[mode][c.wk] != lds) {
      int per_cu = 0;
      const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, lut4_kernel<MT, NG, TPW, D>(mode),
                                                                        (int)block.x, lds);
      if (e != hipSuccess) return e;
      occ[mode][c.wk] = std::max(per_cu, 1);
      occ_lds[mode][c.wk] = lds;
    }
    slots = std::max(1L, (long)cus * occ[mode][c.wk] / MY);
    return hipSuccess;
  };
  // Staged block scales: one batch row, one tile-row of one-group chunks, at
  // most two words per thread (16 G <= 2 threads), room in LDS, and at least
  // two row groups per workgroup (sweeps of the 8B and 70B layers: 70B
  // gate+up at M = 1 54.3 -> 50.2 us, q 14.4 -> 13.7; with one row group
  // per workgroup, or at M = 2, staging cost up to 6%).
  int mode = sal ? 1 : 0;
  size_t lds = total - TABLE_BYTES;  // dynamic part (the table is static)
  long slots = 0;
  bool bs = MT == 1 && NG == 1 && TPW == 1 && sal && 8 * G <= (int)block.x &&
            total + lut4_bs_bytes(a.K) <= LUT4_LDS_LIMIT;
  if (const char* e = tune_env("QGEMV_LUT4_BS")) bs = bs && e[0] != '0';  // tuning override ("0": off)
  if (bs) {
    e0 = slots_of(2, lds + lut4_bs_bytes(a.K), slots);
    if (e0 != hipSuccess) return e0;
    const char* force = tune_env("QGEMV_LUT4_BS");
    if (NRG >= 2 * slots || (force && force[0] == '2')) {  // ("2": regardless of the row groups)
      mode = 2;
      lds += lut4_bs_bytes(a.K);
    }
  }
  if (mode != 2) {
    e0 = slots_of(mode, lds, slots);
    if (e0 != hipSuccess) return e0;
  }
  const dim3 grid((unsigned)std::min<long>(NRG, slots), MY);
  if constexpr (NG == 1 && TPW == 1)
    if (mode == 2) {
      hipLaunchKernelGGL((gemv_lut4_kernel<MT, NG, TPW, D, true, true>), grid, block, lds, s, a);
      return hipGetLastError();
    }
  if (mode == 1)
    hipLaunchKernelGGL((gemv_lut4_kernel<MT, NG, TPW, D, true, false>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((gemv_lut4_kernel<MT, NG, TPW, D, false, false>), grid, block, lds, s, a);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_lm(const Lut4Args& a, const Lut4Cfg& c, hipStream_t s) {
  switch (c.tpw * 100 + c.ng * 10 + (c.tpw >= 2 ? 2 : c.d)) {
    case 112: return launch_l<MT, 1, 1, 2>(a, c, s);
    case 114: return launch_l<MT, 1, 1, 4>(a, c, s);
    case 118: return launch_l<MT, 1, 1, 8>(a, c, s);
    case 122: return launch_l<MT, 2, 1, 2>(a, c, s);
    case 124: return launch_l<MT, 2, 1, 4>(a, c, s);
    case 242: return launch_l<MT, 4, 2, 2>(a, c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t lut4_max_k(int mt) {
  // largest multiple of 128 whose staged rows and table fit with 8 waves x 2 tile-rows
  size_t k = 0;
  while (lut4_lds_bytes(mt, 2, 8, (int)(k + 128)) <= LUT4_LDS_LIMIT) k += 128;
  return k;
}

Lut4Cfg pick_lut4(int M, int N, int K) {
  Lut4Cfg c;
  c.mt = M <= 1 ? 1 : 2;
  if ((size_t)K > lut4_max_k(c.mt)) c.mt = 1;
  const int G = K / 128;
  const long nt = (N + 15) / 16;
  // sweeps on MI355X (Llama-3-8B and 70B layers, M = 1, 2) with the
  // persistent grid: one tile-row per row group and one-group chunks; 8
  // waves with a 4-slot ring once K > 4096, except that narrow layers (at
  // most 256 tile-rows) at M = 1 take 16 waves with 2 slots (4096x4096:
  // 5.9 vs 6.6 us; 4096x14336: 9.6 vs 9.9 us)
  c.tpw = 1;
  c.ng = 1;
  if (c.mt == 1 && nt <= 256 && G >= 16) {
    c.d = 2;
    c.wk = 16;
  } else {
    c.d = K > 4096 ? 4 : 2;
    c.wk = G < 8 ? G : 8;
  }
  return c;
}

hipError_t launch_gemv_lut4(const Lut4Args& a, const Lut4Cfg& c, hipStream_t s) {
  if (c.wk < 1 || c.wk > (c.mt == 1 ? 16 : 8)) return hipErrorInvalidValue;
  switch (c.mt) {
    case 1: return launch_lm<1>(a, c, s);
    case 2: return launch_lm<2>(a, c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
