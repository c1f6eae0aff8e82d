// Prefill-size GEMM over the packed uniform weights: Y = X . dequant(Wq)^T
// for any M (the decode GEMV kernels take M <= 16), on the matrix cores.
//
// The pages' decode kernels turn compute-bound as the batch grows (QFactory
// review, "Key observations": larger batches shift the kernel from memory-
// to compute-bound; ADAngel review: batch growth turns kernels
// compute-bound).  Here the weights stay in their tiled device layout: a
// lane's 32 consecutive k of one row in one quant group are exactly the B
// operand of v_mfma_f32_16x16x32_f16 (as in the decode MFMA engine), so a
// wave dequantizes its B fragments in registers straight from global memory
// and exactly ((q - z) in fp16).  The activations of the block's rows are
// staged in LDS one quant group (128 k) at a time, double-buffered, and
// shared by the workgroup; they go straight from global memory into LDS
// (16-byte buffer loads with an LDS destination), so they occupy no
// registers on the way.
//
// Block: 16 NMT activation rows x 64 NNT weight rows (4 NNT tile-rows), 4
// waves per K half (one or two halves, KH).  Wave w of a half owns
// tile-rows NNT w .. NNT w + NNT - 1 and every
// activation row of the block: each weight fragment is dequantized once per
// workgroup, and each activation fragment read from LDS feeds NNT MFMAs (one
// per tile-row).  NNT = 4 (256 weight rows) quarters the LDS reads per MFMA
// of a one-tile-row-per-wave split (which would ask for about twice the LDS
// bandwidth the matrix cores can use); NNT = 2 (128 weight rows) doubles
// the workgroups of a narrow layer, where 256-row blocks leave one wave per
// SIMD with nothing to overlap its loads, dequantization and MFMAs.  Per
// group a wave runs 4 NMT NNT MFMAs into group partials and adds each times
// its row's scale (one rounding per group, as the decode kernels).  With
// two K halves the halves' partials are added in a fixed order at the end.
// Deterministic.
//
// Block order: workgroups go to the eight XCDs round robin, so consecutive
// ids are renumbered to give each XCD a contiguous range of blocks, with the
// activation blocks of one weight slice adjacent: the XCD's L2 serves that
// slice's weights to all of them.
#include "common.hpp"
#include "dequant.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

constexpr int NXCD = 8;

__device__ __forceinline__ h8 cat4(h2 a, h2 b, h2 c, h2 d) {
  return __builtin_bit_cast(h8, u4{as_u32(a), as_u32(b), as_u32(c), as_u32(d)});
}

// QS: K/128 is a multiple of 8 and the quant params are 16-byte aligned: a
// block's 64 NNT rows of scales and zero-point words are staged in LDS 8
// groups at a time with coalesced 16-byte loads (one row per thread of the
// first NNT waves), instead of per-lane loads that touch 16 rows' cache
// lines for each tile-row and group.
// KH: K halves per workgroup (1 or 2).  With 2, the workgroup has 8 waves:
// waves 4 h .. 4 h + 3 take the groups g = 2 s + h of the block (the same
// tile-rows and activation rows for both halves), each half with its own
// activation buffers; at the end the second half's partials go through LDS
// and the first half adds them in a fixed order.  A narrow layer then keeps
// two waves per SIMD with half the workgroups.
template <int BITS, int NMT, int NNT, bool QS, int KH>
__global__ void __launch_bounds__(256 * KH, 2 / KH) gemm_tiles_kernel(UniformArgs a, int nmb, int nnb) {
  using TR = Uni<BITS>;
  constexpr int PPD = TR::CPD / 2;
  constexpr int ZPW = 32 / BITS;
  constexpr uint32_t ZMASK = (1u << BITS) - 1u;
  constexpr uint32_t TB = 16u * 128u * BITS / 8;  // tile bytes
  constexpr int BM = 16 * NMT;                    // activation rows per block
  // staged activations: [buffer][row][16 pieces of 8 halves], piece c of row
  // r holding k 8 (c ^ (r % 16)) .. + 7 of the group: a row is 256 bytes,
  // so without the swizzle the 16 rows of an A fragment read would all hit
  // the same banks
  // (two separate arrays, selected by a compile-time buffer index: the
  // compiler then knows that reading one never waits for loads into the
  // other)
  // (KH halves: half h uses rows [h BM, h BM + BM) of each buffer)
  __shared__ __attribute__((aligned(16))) _Float16 xs0[KH * BM * 128];
  __shared__ __attribute__((aligned(16))) _Float16 xs1[KH * BM * 128];
  auto xbuf = [&](int b) -> _Float16* { return b ? xs1 : xs0; };
  // staged quant params of an 8-group chunk, two buffers: [row][8] scales and
  // [row][ZW] zero-point words (the words holding the chunk's groups)
  constexpr int ZW = BITS == 8 ? 2 : 1;
  constexpr int BN = 64 * NNT;  // weight rows per block
  __shared__ __attribute__((aligned(16))) uint16_t qs_s[2][QS ? BN * 8 : 8];
  __shared__ __attribute__((aligned(16))) uint32_t qs_z[2][QS ? BN * ZW : 4];

  // (a workgroup past the last block leaves before any barrier)
  const int total = nmb * nnb, per = (total + NXCD - 1) / NXCD;
  const int L = (int)(blockIdx.x % NXCD) * per + (int)(blockIdx.x / NXCD);
  if (L >= total) return;
  const int mb = L % nmb, nb = L / nmb;

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = KH == 1 ? 0 : wid >> 2;  // this wave's K half
  const int wave = KH == 1 ? wid : wid & 3;  // its place among the 4 waves of the half
  const int n = lane & 15, kq = lane >> 4;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / 128;
  const int NT = (N + 15) / 16;
  const uint32_t zrow = 4u * ((G * BITS + 31) / 32);
  const int m0 = mb * BM;
  const int rt0 = nb * 4 * NNT + wave * NNT;  // this wave's first tile-row
  const uint32_t mg = magic1024x2();
  const uint32_t lw = lane_off<BITS>(lane);

  const rsrc_t rw = make_rsrc(a.wq, (uint32_t)NT * G * TB);
  const rsrc_t rz = make_rsrc(a.zeros, (uint32_t)N * zrow);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * G * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);

  // Every load below is unconditional and takes its group (and block-row
  // step) in the scalar offset: rows past M or N and tile-rows past the last
  // fall outside their buffer and read zeros; the stage loaded past the last
  // group is never used.
  //
  // activation staging: wave w fills rows 4 (4 j + w) .. + 3 of the block
  // (j < NMT), one 1 KB load each: lane l writes piece l % 16 of row
  // 4 (4 j + w) + l / 16, i.e. k 8 ((l % 16) ^ (row % 16)) .. + 7.
  const int xr0 = 4 * wave + (lane >> 4);  // the lane's row for j = 0 (row % 16 is the same for every j)
  const uint32_t xbase = ((uint32_t)(m0 + xr0) * K + 8u * (uint32_t)((lane & 15) ^ xr0)) * 2u;
  auto x_issue = [&](int g, int b) {
#pragma unroll
    for (int j = 0; j < NMT; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)&xbuf(b)[(half * 4 * NMT + 4 * j + wave) * 512],
                                               16, xbase, 32u * (uint32_t)K * j + 256u * g, 0, 0);
  };
  // the wave's weights in group g: codes, scale and zero point of lane row n
  // of each of its tile-rows
  struct Wst {
    LaneCodes<BITS> c[NNT];
    uint16_t s[QS ? 1 : NNT];
    uint32_t z[QS ? 1 : NNT];
  };
  const uint32_t soff_n = 2u * (uint32_t)G * n, zoff_n = zrow * n;
  auto w_load = [&](int g, Wst& st) {
#pragma unroll
    for (int t = 0; t < NNT; ++t) {
      const uint32_t rt = (uint32_t)(rt0 + t);
      st.c[t].load(rw, lw, (rt * G + g) * TB);
      if constexpr (!QS) {
        st.s[t] = bload2(rs, soff_n, 32u * G * rt + 2u * g);
        st.z[t] = bload4(rz, zoff_n, 16u * zrow * rt + 4u * (uint32_t)(g / ZPW));
      }
    }
  };
  // the staged quant params of chunk c (groups 8c .. 8c + 7): thread t < BN
  // loads block row t's 8 scales and its zero-point words (with NNT = 2 the
  // last two waves stage nothing: a wave-uniform branch)
  const bool qwave = wid < NNT;
  const uint32_t qrow = (uint32_t)nb * BN + threadIdx.x;
  const uint32_t qs_v = qrow * (uint32_t)G * 2u, qz_v = qrow * zrow;
  auto q_issue = [&](int c, u4& sv, uint32_t (&zv)[ZW]) {
    if (!qwave) return;
    sv = bload16(rs, qs_v, 16u * (uint32_t)c);
#pragma unroll
    for (int e = 0; e < ZW; ++e) zv[e] = bload4(rz, qz_v, 4u * ((uint32_t)(8 * c) / ZPW + e));
  };
  auto q_store = [&](int b, const u4& sv, const uint32_t (&zv)[ZW]) {
    if (!qwave) return;
    *reinterpret_cast<u4*>(&qs_s[b][threadIdx.x * 8]) = sv;
#pragma unroll
    for (int e = 0; e < ZW; ++e) qs_z[b][threadIdx.x * ZW + e] = zv[e];
  };

  f4 acc[NMT][NNT];
#pragma unroll
  for (int i = 0; i < NMT; ++i)
#pragma unroll
    for (int t = 0; t < NNT; ++t) acc[i][t] = f4{0.f, 0.f, 0.f, 0.f};

  // Tile-row-major: the A fragments of every activation tile are read once
  // (NMT x 4 registers of 16 bytes), then each tile-row's MFMAs are issued
  // interleaved with the dequantization of the next tile-row (independent
  // work the compiler schedules between the MFMAs).
  auto compute = [&](int g, int b, const Wst& st) {
    u4 av[NMT][4];
#pragma unroll
    for (int i = 0; i < NMT; ++i) {
      // block row 16 i + n, k 32 kq + 8 s .. + 7 of the group
      const u4* xr = reinterpret_cast<const u4*>(&xbuf(b)[(half * BM + 16 * i + n) * 128]);
#pragma unroll
      for (int s = 0; s < 4; ++s) av[i][s] = xr[(4 * kq + s) ^ n];
    }
    // B fragments: the (q - z) pairs of the lane's 32 k in tile-row t
    // quant params of tile-row t in group g: the lane's row, from the staged
    // chunk or from the stage's own loads
    const int cb = (g >> 3) & 1, lr0 = 16 * wave * NNT + n;
    auto zword = [&](int t) -> uint32_t {
      if constexpr (QS) return qs_z[cb][(lr0 + 16 * t) * ZW + ((g & 7) * BITS) / 32];
      else return st.z[t];
    };
    auto scale = [&](int t) -> uint16_t {
      if constexpr (QS) return qs_s[cb][(lr0 + 16 * t) * 8 + (g & 7)];
      else return st.s[t];
    };
    auto deq_t = [&](int t, h2 (&p)[16]) {
      const typename TR::Z zz = TR::zc((zword(t) >> (BITS * (g % ZPW))) & ZMASK);
#pragma unroll
      for (int d = 0; d < BITS; ++d) TR::deq(st.c[t].w[d], mg, zz, p + d * PPD);
    };
    h2 p[2][16];
    deq_t(0, p[0]);
#pragma unroll
    for (int t = 0; t < NNT; ++t) {
      if (t + 1 < NNT) deq_t(t + 1, p[(t + 1) & 1]);
      const float sc = h2f(scale(t));
#pragma unroll
      for (int i = 0; i < NMT; ++i) {
        f4 dd = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(h8, av[i][s]),
              cat4(p[t & 1][4 * s], p[t & 1][4 * s + 1], p[t & 1][4 * s + 2], p[t & 1][4 * s + 3]), dd, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][t][r] = fmaf(sc, dd[r], acc[i][t][r]);
      }
    }
  };

  // Pipeline: group g is computed from LDS buffer g % 2 and register stage
  // g % 2.  At the start of a step the activations of group g + 1 go into the
  // other buffer (every wave is past group g - 1, its last reader), then the
  // weights of group g + 1 into the other register stage; at its end the
  // wave waits for its activation loads only (loads complete in order), and
  // the barrier for every wave's.  Loads past the last group read zeros.
  // WLOADS: the vector memory instructions of one w_load.
  constexpr int WLOADS = NNT * ((BITS == 8 ? 2 : 1) + (QS ? 0 : 2));
  static_assert(WLOADS < 64, "vmcnt range");
  constexpr int VMW = (WLOADS & 15) | (0x7 << 4) | (0xF << 8) | ((WLOADS >> 4) << 14);  // s_waitcnt vmcnt(WLOADS)
  Wst wst[2];
  u4 qsv;
  uint32_t qzv[ZW];
  if constexpr (QS) {
    q_issue(0, qsv, qzv);
    q_store(0, qsv, qzv);  // (waits for these loads only)
  }
  x_issue(half, 0);
  __builtin_amdgcn_sched_barrier(0);
  w_load(half, wst[0]);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(VMW);
  lds_barrier();

  // (the scheduling barriers keep the loads at the start of the step, in
  // this order, where the compiler would sink them to the end to save
  // registers)
  auto step = [&](int g, int b, const Wst& cur, Wst& next) {
    // the last step of a chunk also stages the next chunk's quant params
    // (into the other buffer: its previous chunk was last read a whole
    // chunk ago, before several barriers); with two K halves a step covers
    // groups g - half and g - half + 1, which share a chunk (8 | K/128)
    const int gn = g - half + KH;  // the first group of the next step
    const bool qnext = QS && (gn & 7) == 0 && gn < G;
    if constexpr (QS)
      if (qnext) q_issue(gn >> 3, qsv, qzv);
    __builtin_amdgcn_sched_barrier(0);
    x_issue(g + KH, b ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    w_load(g + KH, next);
    __builtin_amdgcn_sched_barrier(0);
    compute(g, b, cur);
    if constexpr (QS)
      if (qnext) q_store((gn >> 3) & 1, qsv, qzv);
    __builtin_amdgcn_s_waitcnt(VMW);  // this wave's activation loads of group g + 1
    lds_barrier();
  };
  // two groups per iteration so the register stages are named statically
  // (every wave runs the same number of steps; a half's group past the last
  // reads zeros)
  const int S = (G + KH - 1) / KH;
  for (int st = 0; st < S; st += 2) {
    step(KH * st + half, 0, wst[0], wst[1]);
    if (st + 1 < S) step(KH * (st + 1) + half, 1, wst[1], wst[0]);
  }
  if constexpr (KH == 2) {
    // the second half's partials into LDS (over the activation buffers:
    // every load into them has landed and every read is done, the last
    // step ended with a barrier), then added by the first half
    float* red = reinterpret_cast<float*>(xs0);
    constexpr int NV = NMT * NNT * 4;
    if (half == 1) {
#pragma unroll
      for (int i = 0; i < NMT; ++i)
#pragma unroll
        for (int t = 0; t < NNT; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[((wave * NV) + (i * NNT + t) * 4 + r) * 64 + lane] = acc[i][t][r];
    }
    lds_barrier();
    if (half == 1) return;
#pragma unroll
    for (int i = 0; i < NMT; ++i)
#pragma unroll
      for (int t = 0; t < NNT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][t][r] += red[((wave * NV) + (i * NNT + t) * 4 + r) * 64 + lane];
  }

  // lane l holds D[row 4 (l / 16) + r][weight row l % 16] of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < NMT; ++i)
#pragma unroll
    for (int t = 0; t < NNT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * i + 4 * kq + r;
        const int row = 16 * (rt0 + t) + n;
        if (m < M && row < N) a.y[(size_t)m * N + row] = f2h(acc[i][t][r]);
      }
}

}  // namespace

template <int BITS, int NMT, int NNT, int KH = 1>
hipError_t launch_bm(const UniformArgs& a, hipStream_t s) {
  const int NT = (a.N + 15) / 16;
  const int nmb = (a.M + 16 * NMT - 1) / (16 * NMT);
  const int nnb = (NT + 4 * NNT - 1) / (4 * NNT);
  const long total = (long)nmb * nnb;
  const long grid = (total + NXCD - 1) / NXCD * NXCD;
  if (grid > 0x7FFFFFFFL) return hipErrorInvalidValue;
  const bool qs = (a.K / 128) % 8 == 0 && reinterpret_cast<uintptr_t>(a.scales) % 16 == 0;
  if (qs)
    hipLaunchKernelGGL((gemm_tiles_kernel<BITS, NMT, NNT, true, KH>), dim3((unsigned)grid), dim3(256 * KH), 0, s, a, nmb, nnb);
  else
    hipLaunchKernelGGL((gemm_tiles_kernel<BITS, NMT, NNT, false, KH>), dim3((unsigned)grid), dim3(256 * KH), 0, s, a, nmb, nnb);
  return hipGetLastError();
}

// mi: 16-row activation tiles per block (2: 32-row blocks, 4: 64-row
// blocks); nt: tile-rows per wave (4: 256-column blocks, 2: 128-column
// blocks).  8-bit weights take 32-row blocks either way: two register
// stages of their codes and the partials of 64 rows do not fit the 256
// registers of two waves per SIMD.
template <int BITS>
hipError_t launch_bits(const UniformArgs& a, int mi, int nt, int kh, hipStream_t s) {
  if (kh == 2) {  // (two K halves: the 128-column blocks)
    if (nt != 2) return hipErrorInvalidValue;
    if constexpr (BITS != 8)
      if (mi == 4) return launch_bm<BITS, 4, 2, 2>(a, s);
    return launch_bm<BITS, 2, 2, 2>(a, s);
  }
  if constexpr (BITS != 8)
    if (mi == 4) return nt == 4 ? launch_bm<BITS, 4, 4>(a, s) : launch_bm<BITS, 4, 2>(a, s);
  return nt == 4 ? launch_bm<BITS, 2, 4>(a, s) : launch_bm<BITS, 2, 2>(a, s);
}

hipError_t launch_gemm_tiles(const UniformArgs& a, int mi, int nt, int kh, hipStream_t s) {
  if ((mi != 2 && mi != 4) || (nt != 2 && nt != 4) || (kh != 1 && kh != 2)) return hipErrorInvalidValue;
  switch (a.bits) {
    case 2: return launch_bits<2>(a, mi, nt, kh, s);
    case 4: return launch_bits<4>(a, mi, nt, kh, s);
    case 8: return launch_bits<8>(a, mi, nt, kh, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
