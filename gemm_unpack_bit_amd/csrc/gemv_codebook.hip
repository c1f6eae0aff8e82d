// Codebook GEMV with a Psumbook (m = 1 codebook of 256 centroids, v = 4,
// b = 8, one fp16 scale per 128 k), at decode batch M <= 16, on gfx950:
//
//   w[n, 4j + t] = s[n, (4j + t) / 128] * C[code[n, j]][t]
//   P[m][j][c]   = sum_t C[c][t] * x[m, 4j + t]                (Psumbook)
//   y[m, n]      = sum_G s[n, G] * sum_{j in G} P[m][j][code[n, j]]
//
// The CodeGEMM paper notes: instead of dequantizing, precompute the partial
// sums of every centroid with every v-wide activation segment once, keep them
// on chip, and accumulate outputs by code lookup; the build is amortized over
// many weight rows.
//
// Design (gfx950):
//  * Codes are an [N, K/4] uint8 matrix in the 64-row layout
//    (qgemv_pack(8, QGEMV_LAYOUT_ROWS64, N, K/4)): a 1 KB tile holds 16
//    consecutive codes of 64 rows, lane l of a wave-wide 16-byte load getting
//    its own row's 16 codes.  A "pair" of 2 quant groups (64 segments, 256 k)
//    is 4 consecutive tiles of a row block, 4 KB contiguous.
//  * Psumbook of a pair in LDS, segment-major: fp16 P[s][c] at byte
//    520 s + 2 c (33 KB, so 4 workgroups share a CU and keep its LDS busy
//    while one of them waits at a barrier).  All lanes of a wave look up the
//    same segment s at once, so s is the instruction's immediate offset and
//    the lane address is 2 * code; the bank follows the (random) code, not the
//    segment.  Two lookups are summed into the fp32 partial by one v_dot2
//    against (1, 1).  Each lane owns one weight row, so no cross-lane
//    reduction is needed.  The random 64-lane lookups are the bound: the LDS
//    serves one about every 3 to 4 clocks per CU.
//  * Build on the matrix cores: one v_mfma_f32_32x32x8_f16 gives P for 32
//    centroids x 32 segments (A = codebook rows, B = activation segments, the
//    v = 4 dims padded to 8 with zeros); 16 of them per pair, spread over the
//    waves of the workgroup.  Each lane then holds 4 consecutive centroids of
//    one segment per register quartet and writes them with one 8-byte store;
//    the segment rows are 520 bytes apart (256 fp16 + 8 bytes of padding), so
//    the 32 segments of a store land in distinct banks.  Each wave keeps the
//    codebook rows it multiplies in registers for the whole kernel.
//  * Three kernels share this design.  The stationary kernel gives each
//    workgroup one K part (1, 2 or 4 pairs) and streams many row blocks
//    through its Psumbook, built once, with no barrier after the build.  The
//    batched stationary kernel (M >= 2) stores the partial sums of 2 or 4
//    batch rows in each Psumbook entry, so one lookup serves them all.  The
//    sequential kernel gives each workgroup WK row blocks and a K range, and
//    per pair runs LDS barrier / build / LDS barrier / lookups, with the next
//    pair's codes, scales and activation segments in flight meanwhile (the
//    barriers wait for LDS traffic only); it serves small layers and calls
//    without a workspace.
//  * K parts write fp32 partial sums to the caller's workspace and a second,
//    small kernel adds the parts of every output in a fixed order, so the
//    result is deterministic and no workgroup waits on another.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

constexpr uint32_t PSTRIDE = 520u;              // bytes per segment row: 256 fp16 + 8 of padding
constexpr uint32_t PSUM_BYTES = 64u * PSTRIDE;  // the Psumbook of one pair

typedef _Float16 h4v __attribute__((ext_vector_type(4)));

// NSB: activation segment blocks each wave multiplies per pair (2 / min(WK, 2)).
// SAL: the scales base is 4-byte aligned, so a pair's 2 scales of a row are
// one load (K is a multiple of 512, so every row's pair starts 4-aligned too).
template <int NSB, bool SAL>
__global__ void __launch_bounds__(NSB == 1 ? 1024 : 64) gemv_codebook_seq_kernel(CodebookArgs a) {
  __shared__ __attribute__((aligned(16))) uint32_t lsm[PSUM_BYTES / 4];
  char* const lds = reinterpret_cast<char*>(lsm);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int WK = blockDim.x >> 6;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / 128;   // quant groups
  const int HN = K / 256;  // pairs
  const int NCB = K / 64;  // 16-code tiles per row block
  const int NB = (N + 63) / 64;
  const int m = blockIdx.z;
  const int ks = blockIdx.y, KS = gridDim.y;
  const int h0 = (HN * ks) / KS, h1 = (HN * (ks + 1)) / KS;
  const int rb = blockIdx.x * WK + wave;  // this wave's 64-row block
  const uint32_t row = (uint32_t)rb * 64u + lane;
  const bool rv = rb < NB && row < (uint32_t)N;

  const rsrc_t rc = make_rsrc(a.codes, (uint32_t)NB * NCB * 1024u);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * G * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);

  struct St {
    u4 c[4];        // 4 tiles x 16 codes of this lane's row
    uint16_t s[2];  // the pair's 2 group scales of this row
  };
  // Loads are unconditional, with every choice in the offsets: a wave past
  // the last row block reads zero codes, a row past N zero scales.  The
  // prefetch past the K range re-reads the range's last pair (never used),
  // so that the pair index only ever moves the wave-uniform offsets.
  const uint32_t vcode = rb < NB ? 16u * lane : OOB;
  const uint32_t vscale = rv ? row * (uint32_t)G * 2u : OOB;
  auto load_stage = [&](int h, St& st) {
    const uint32_t hc = (uint32_t)min(h, h1 - 1);
    const uint32_t sw = __builtin_amdgcn_readfirstlane(((uint32_t)min(rb, NB - 1) * NCB + 4u * hc) * 1024u);
#pragma unroll
    for (int i = 0; i < 4; ++i) st.c[i] = bload16<CPOL_NT>(rc, vcode + 1024u * i, sw);
    if constexpr (SAL) {
      const uint32_t v = bload4(rs, vscale, 4u * hc);
      st.s[0] = (uint16_t)v;
      st.s[1] = (uint16_t)(v >> 16);
    } else {
#pragma unroll
      for (int g = 0; g < 2; ++g) st.s[g] = bload2(rs, vscale, 4u * hc + 2u * g);
    }
  };

  // Build assignment: the 16 MFMA blocks of a pair are 2 segment blocks (sb)
  // x 8 centroid blocks (cb).  With W2 = min(WK, 2) and WC = max(WK / 2, 1),
  // wave w takes sb = w % 2 + j W2 (j < NSB) and cb = w / 2 + c WC
  // (c < 8 / WC): 16 / WK blocks, each block exactly once.
  const int W2 = WK < 2 ? WK : 2;
  const int WC = WK < 2 ? 1 : WK / 2;
  const int NCW = 8 / WC;  // centroid blocks per wave
  const int li = lane & 31;
  const bool klo = lane < 32;  // lanes holding dims 0..3 (the others: the zero padding)

  // A operands: codebook rows 32 cb + l % 32 of this wave's centroid blocks
  h4v ca[8];
  {
    const rsrc_t rcb = make_rsrc(a.codebook, 256u * 8u);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t cb = (uint32_t)((wave >> 1) + c * WC);
      const uint32_t v = klo && c < NCW ? (32u * cb + li) * 8u : OOB;
      ca[c] = __builtin_bit_cast(h4v, __builtin_amdgcn_raw_buffer_load_b64(rcb, v, 0, 0));
    }
  }
  // B operands: segment 32 sb + l % 32 of pair h, 4 halves
  uint32_t vx[NSB];
#pragma unroll
  for (int j = 0; j < NSB; ++j) vx[j] = klo ? ((uint32_t)m * K + 4u * (32u * ((wave & 1) + j * W2) + li)) * 2u : OOB;
  struct Xs {
    u2 v[NSB];
  };
  auto load_xs = [&](int h, Xs& xs) {
    const uint32_t hc = (uint32_t)min(h, h1 - 1);
#pragma unroll
    for (int j = 0; j < NSB; ++j)
      xs.v[j] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rx, vx[j], 512u * hc, 0));
  };
  // this lane's store address within a segment block: segment l % 32, the
  // 4-centroid quartet 4 (l / 32) of each 8-centroid group
  const uint32_t pw = (uint32_t)li * PSTRIDE + 8u * (uint32_t)(lane >> 5);

  St ring[2];
  Xs xr[2];
  load_stage(h0, ring[0]);
  load_xs(h0, xr[0]);

  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  float acc = 0.f;

  auto step = [&](int h, const St& st, St& nxt, const Xs& xs, Xs& xn) {
    load_stage(h + 1, nxt);  // next pair (past the range: a harmless re-read)
    load_xs(h + 1, xn);
    lds_barrier();  // every wave is done reading the previous pair's P
#pragma unroll
    for (int j = 0; j < NSB; ++j) {
      const uint32_t sb = (uint32_t)((wave & 1) + j * W2);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (c >= NCW) break;
        const uint32_t cb = (uint32_t)((wave >> 1) + c * WC);
        const f16v d = __builtin_amdgcn_mfma_f32_32x32x8f16(ca[c], __builtin_bit_cast(h4v, xs.v[j]), f16v{}, 0, 0, 0);
        // lane l, register 4 g + i: P[32 sb + l % 32][32 cb + 8 g + 4 (l / 32) + i]
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const h4v hv = {(_Float16)d[4 * g], (_Float16)d[4 * g + 1], (_Float16)d[4 * g + 2], (_Float16)d[4 * g + 3]};
          *reinterpret_cast<u2*>(lds + pw + sb * (32u * PSTRIDE) + 64u * cb + 16u * g) = __builtin_bit_cast(u2, hv);
        }
      }
    }
    lds_barrier();  // P of this pair complete
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float part = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {  // tile 2g + t: segments 32g + 16t + 0..15
#pragma unroll
        for (int d = 0; d < 4; ++d) {  // word d: segments 32g + 16t + 4d + 0..3
          const uint32_t w = st.c[2 * g + t][d];
          const uint32_t s0 = 32u * g + 16u * t + 4u * d;
          h2 pa, pb;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t code2 = __builtin_amdgcn_ubfe(w, 8 * b, 8) << 1;
            const _Float16 v = *reinterpret_cast<const _Float16*>(lds + code2 + PSTRIDE * (s0 + b));
            if (b < 2)
              pa[b] = v;
            else
              pb[b - 2] = v;
          }
          part = dot2(pa, ones, part);
          part = dot2(pb, ones, part);
        }
      }
      acc = fmaf(h2f(st.s[g]), part, acc);
    }
  };
  // two pairs per iteration so the stage buffers are named statically
  for (int h = h0; h < h1; h += 2) {
    step(h, ring[0], ring[1], xr[0], xr[1]);
    if (h + 1 < h1) step(h + 1, ring[1], ring[0], xr[1], xr[0]);
  }

  if (!rv) return;
  if (KS == 1)
    a.y[(size_t)m * N + row] = f2h(acc);
  else  // K split: this range's partial sum, added up by the reduce kernel
    a.ws[((size_t)ks * M + m) * N + row] = acc;
}

// Stationary kernel: a workgroup owns one K part of PP pairs (SEG = 64 PP
// segments) and one batch row, builds that part's Psumbook once, and streams
// row blocks through it: wave w of row slice r takes row blocks
// r WK + w + i R WK.  There is no barrier after the build, so every wave
// runs at its own pace and the lookups of the 16 waves on a CU keep the LDS
// busy.  Each part writes fp32 partial sums; the reduce kernel adds them.
//
// Grid: one dimension of 8 * ceil(R * KP / 8) * M workgroups.  Workgroup b
// takes batch row m = (b / 8) % M and unit u = (b / (8 M)) * 8 + b % 8
// (row slice u % R, K part u / R), so the M workgroups that read the same
// codes get ids b, b + 8, ..., which are dispatched together and to the same
// XCD (ids are dealt to the 8 XCDs in turn), and share its L2.  (Running the
// K parts of a row slice together instead, so that neighbours read adjacent
// 4 KB runs, measured slower.)
template <int PP, bool SAL>
__global__ void __launch_bounds__(PP == 4 ? 512 : 1024) gemv_codebook_stat_kernel(CodebookArgs a, int R) {
  constexpr uint32_t SEG = 64u * PP;
  constexpr uint32_t PBYTES = SEG * PSTRIDE;
  // LDS: [Psumbook SEG x 520 B][codebook 256 x 8 B][activation segments SEG x 8 B]
  __shared__ __attribute__((aligned(16))) uint32_t lsm[(PBYTES + 2048u + SEG * 8u) / 4];
  char* const lds = reinterpret_cast<char*>(lsm);
  u2* const stg = reinterpret_cast<u2*>(lds + PBYTES);  // codebook rows, then the segments

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int WK = blockDim.x >> 6;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / 128;   // quant groups
  const int NCB = K / 64;  // 16-code tiles per row block
  const int NB = (N + 63) / 64;
  const int KP = K / (256 * PP);
  const uint32_t b = blockIdx.x;
  const int m = (int)((b >> 3) % (uint32_t)M);
  const uint32_t u = (b / (8u * (uint32_t)M)) * 8u + (b & 7u);
  if (u >= (uint32_t)R * (uint32_t)KP) return;  // padding: the whole workgroup
  const int r = (int)(u % (uint32_t)R), kp = (int)(u / (uint32_t)R);

  const int RS = R * WK;
  const int rb0 = r * WK + wave;
  const int cnt = rb0 < NB ? (NB - 1 - rb0) / RS + 1 : 0;  // this wave's row blocks

  const rsrc_t rc = make_rsrc(a.codes, (uint32_t)NB * NCB * 1024u);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * G * 2u);

  struct St {
    u4 c[4 * PP];     // 4 PP tiles x 16 codes of this lane's row
    uint32_t s[PP];   // the part's 2 PP group scales of this row, two per word
  };
  // Unconditional loads, every choice in the offsets: past this wave's last
  // row block (and for a row past N) the offsets are out of range, so the
  // loads return zeros without touching memory.
  auto load_stage = [&](int i, St& st) {
    const bool bv = i < cnt;
    const int rb = rb0 + i * RS;
    const uint32_t sw =
        __builtin_amdgcn_readfirstlane(((uint32_t)(bv ? rb : 0) * NCB + 4u * PP * (uint32_t)kp) * 1024u);
    const uint32_t vc = bv ? 16u * lane : OOB;
#pragma unroll
    for (int j = 0; j < 4 * PP; ++j) st.c[j] = bload16<CPOL_NT>(rc, vc + 1024u * j, sw);
    const uint32_t row = (uint32_t)rb * 64u + lane;
    const uint32_t vs = bv && row < (uint32_t)N ? (row * (uint32_t)G + 2u * PP * (uint32_t)kp) * 2u : OOB;
#pragma unroll
    for (int j = 0; j < PP; ++j) {
      if constexpr (SAL)
        st.s[j] = bload4(rs, vs + 4u * j);
      else
        st.s[j] = (uint32_t)bload2(rs, vs + 4u * j) | ((uint32_t)bload2(rs, vs + 4u * j + 2u) << 16);
    }
  };

  // The codebook and this part's activation segments (256 + SEG 8-byte
  // entries, at most 8 per thread) are loaded first: a wave's loads return in
  // order, so the build then waits for these only, not for the code prefetch
  // issued after them.
  u2 sv[8];
  {
    const rsrc_t rcb = make_rsrc(a.codebook, 2048u);
    const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = threadIdx.x + j * (int)blockDim.x;
      const uint32_t xo = ((uint32_t)m * K + 4u * (SEG * (uint32_t)kp + (uint32_t)(i - 256))) * 2u;
      sv[j] = i < 256 ? __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rcb, 8u * i, 0, 0))
                      : __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(
                                                   rx, i < 256 + (int)SEG ? xo : OOB, 0, 0));
    }
  }
  // D row blocks of codes per wave: D - 1 in flight during the lookups of one
  constexpr int D = PP == 1 ? 4 : (PP == 2 ? 3 : 2);
  St ring[D];
#pragma unroll
  for (int k = 0; k + 1 < D; ++k) load_stage(k, ring[k]);  // in flight during the build
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = threadIdx.x + j * (int)blockDim.x;
    if (i < 256 + (int)SEG) stg[i] = sv[j];
  }
  __syncthreads();
  // Build: 2 PP segment blocks x 8 centroid blocks, one v_mfma_f32_32x32x8_f16
  // each (A = codebook rows, B = activation segments, dims 4..7 zero)
  {
    const int li = lane & 31;
    const bool klo = lane < 32;
    const uint32_t pw = (uint32_t)li * PSTRIDE + 8u * (uint32_t)(lane >> 5);
    for (int p = wave; p < 16 * PP; p += WK) {
      const uint32_t sb = (uint32_t)(p % (2 * PP)), cb = (uint32_t)(p / (2 * PP));
      const u2 av = stg[32u * cb + li], bv = stg[256u + 32u * sb + li];
      const u2 A = {klo ? av.x : 0u, klo ? av.y : 0u}, B = {klo ? bv.x : 0u, klo ? bv.y : 0u};
      const f16v d = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(h4v, A), __builtin_bit_cast(h4v, B), f16v{},
                                                          0, 0, 0);
      // lane l, register 4 g + i: P[32 sb + l % 32][32 cb + 8 g + 4 (l / 32) + i]
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const h4v hv = {(_Float16)d[4 * g], (_Float16)d[4 * g + 1], (_Float16)d[4 * g + 2], (_Float16)d[4 * g + 3]};
        *reinterpret_cast<u2*>(lds + pw + sb * (32u * PSTRIDE) + 64u * cb + 16u * g) = __builtin_bit_cast(u2, hv);
      }
    }
  }
  __syncthreads();

  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  auto step = [&](int i, const St& st, St& nxt) {
    load_stage(i + D - 1, nxt);  // a later row block (past the last: a harmless re-read)
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < 2 * PP; ++g) {
      float part = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {  // tile 2g + t: segments 32g + 16t + 0..15
#pragma unroll
        for (int d = 0; d < 4; ++d) {  // word d: segments 32g + 16t + 4d + 0..3
          const uint32_t w = st.c[2 * g + t][d];
          const uint32_t s0 = 32u * g + 16u * t + 4u * d;
          h2 pa, pb;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const uint32_t code2 = __builtin_amdgcn_ubfe(w, 8 * bb, 8) << 1;
            const _Float16 v = *reinterpret_cast<const _Float16*>(lds + code2 + PSTRIDE * (s0 + bb));
            if (bb < 2)
              pa[bb] = v;
            else
              pb[bb - 2] = v;
          }
          part = dot2(pa, ones, part);
          part = dot2(pb, ones, part);
        }
      }
      acc = fmaf(h2f((uint16_t)(st.s[g / 2] >> (16 * (g % 2)))), part, acc);
    }
    const uint32_t row = (uint32_t)(rb0 + i * RS) * 64u + lane;
    if (row < (uint32_t)N) {
      if (KP == 1)
        a.y[(size_t)m * N + row] = f2h(acc);
      else
        a.ws[((size_t)kp * M + m) * N + row] = acc;
    }
  };
  // D row blocks per iteration so the stage buffers are named statically
  for (int i = 0; i < cnt; i += D) {
#pragma unroll
    for (int k = 0; k < D; ++k)
      if (i + k < cnt) step(i + k, ring[k], ring[(k + D - 1) % D]);
  }
}

// Batched stationary kernel (M >= 2): as the stationary kernel, but one
// Psumbook serves MB batch rows: entry (s, c) holds the MB rows' partial sums
// as consecutive fp16 (2 MB bytes), so one 4- or 8-byte LDS read per code
// serves every row of the batch block, and the lookups no longer scale with
// M.  Each row's value is added to its fp32 partial by one v_dot2 against a
// unit pair.  Segment rows are 512 MB + 16 bytes apart: the build's 16-byte
// stores of 32 segments spread over the banks.  Batch rows past M read zero
// activations and are not stored.
template <int MB, int PP, bool SAL>
__global__ void __launch_bounds__(512) gemv_codebook_statb_kernel(CodebookArgs a, int R) {
  constexpr uint32_t SEG = 64u * PP;
  constexpr uint32_t EB = 2u * MB;              // bytes per entry
  constexpr uint32_t BS = 256u * EB + 16u;      // bytes per segment row
  constexpr uint32_t PBYTES = SEG * BS;
  constexpr uint32_t SB = 65535u / BS + 1u;     // segments whose offsets fit the 16-bit immediate
  // LDS: [Psumbook SEG x BS][codebook 256 x 8 B][activation segments MB x SEG x 8 B]
  __shared__ __attribute__((aligned(16))) uint32_t lsm[(PBYTES + 2048u + MB * SEG * 8u) / 4];
  char* const lds = reinterpret_cast<char*>(lsm);
  u2* const stg = reinterpret_cast<u2*>(lds + PBYTES);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int WK = blockDim.x >> 6;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / 128;
  const int NCB = K / 64;
  const int NB = (N + 63) / 64;
  const int KP = K / (256 * PP);
  const int MBLK = (M + MB - 1) / MB;
  const uint32_t b = blockIdx.x;
  const int mb = (int)((b >> 3) % (uint32_t)MBLK);
  const uint32_t u = (b / (8u * (uint32_t)MBLK)) * 8u + (b & 7u);
  if (u >= (uint32_t)R * (uint32_t)KP) return;  // padding: the whole workgroup
  const int r = (int)(u % (uint32_t)R), kp = (int)(u / (uint32_t)R);
  const int m0 = mb * MB;

  const int RS = R * WK;
  const int rb0 = r * WK + wave;
  const int cnt = rb0 < NB ? (NB - 1 - rb0) / RS + 1 : 0;

  const rsrc_t rc = make_rsrc(a.codes, (uint32_t)NB * NCB * 1024u);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * G * 2u);

  struct St {
    u4 c[4 * PP];
    uint32_t s[PP];
  };
  auto load_stage = [&](int i, St& st) {
    const bool bv = i < cnt;
    const int rb = rb0 + i * RS;
    const uint32_t sw =
        __builtin_amdgcn_readfirstlane(((uint32_t)(bv ? rb : 0) * NCB + 4u * PP * (uint32_t)kp) * 1024u);
    const uint32_t vc = bv ? 16u * lane : OOB;
#pragma unroll
    for (int j = 0; j < 4 * PP; ++j) st.c[j] = bload16<CPOL_NT>(rc, vc + 1024u * j, sw);
    const uint32_t row = (uint32_t)rb * 64u + lane;
    const uint32_t vs = bv && row < (uint32_t)N ? (row * (uint32_t)G + 2u * PP * (uint32_t)kp) * 2u : OOB;
#pragma unroll
    for (int j = 0; j < PP; ++j) {
      if constexpr (SAL)
        st.s[j] = bload4(rs, vs + 4u * j);
      else
        st.s[j] = (uint32_t)bload2(rs, vs + 4u * j) | ((uint32_t)bload2(rs, vs + 4u * j + 2u) << 16);
    }
  };

  // codebook rows and the MB rows' activation segments first (loads return in
  // order, so the build waits for these only), then the code prefetch
  constexpr int NST = (256 + MB * (int)SEG + 63) / 64;  // staged entries per thread at 64 threads
  u2 sv[NST];
  {
    const rsrc_t rcb = make_rsrc(a.codebook, 2048u);
    const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);
#pragma unroll
    for (int j = 0; j < NST; ++j) {
      const int i = threadIdx.x + j * (int)blockDim.x;
      const int e = i - 256, m = e / (int)SEG, sg = e - m * (int)SEG;
      const bool xv = i >= 256 && i < 256 + MB * (int)SEG && m0 + m < M;
      const uint32_t xo = xv ? ((uint32_t)(m0 + m) * K + 4u * (SEG * (uint32_t)kp + (uint32_t)sg)) * 2u : OOB;
      sv[j] = i < 256 ? __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rcb, 8u * i, 0, 0))
                      : __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rx, xo, 0, 0));
    }
  }
  constexpr int D = PP == 1 ? 4 : 3;
  St ring[D];
#pragma unroll
  for (int k = 0; k + 1 < D; ++k) load_stage(k, ring[k]);
#pragma unroll
  for (int j = 0; j < NST; ++j) {
    const int i = threadIdx.x + j * (int)blockDim.x;
    if (i < 256 + MB * (int)SEG) stg[i] = sv[j];
  }
  __syncthreads();
  // Build: 2 PP segment blocks x 8 centroid blocks, MB v_mfma_f32_32x32x8_f16
  // each (one per batch row); lane l then holds, per register quartet g, 4
  // consecutive centroids x MB rows = 8 MB contiguous bytes of one segment
  {
    const int li = lane & 31;
    const bool klo = lane < 32;
    const uint32_t pw = (uint32_t)li * BS + 4u * EB * (uint32_t)(lane >> 5);
    for (int p = wave; p < 16 * PP; p += WK) {
      const uint32_t sb = (uint32_t)(p % (2 * PP)), cb = (uint32_t)(p / (2 * PP));
      const u2 av = stg[32u * cb + li];
      const u2 A = {klo ? av.x : 0u, klo ? av.y : 0u};
      f16v d[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        const u2 bv = stg[256u + (uint32_t)m * SEG + 32u * sb + li];
        const u2 B = {klo ? bv.x : 0u, klo ? bv.y : 0u};
        d[m] = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(h4v, A), __builtin_bit_cast(h4v, B), f16v{}, 0,
                                                    0, 0);
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        char* const dst = lds + pw + sb * (32u * BS) + (32u * cb + 8u * g) * EB;
        // centroid i of the quartet, row m: half i MB + m
        _Float16 hv[4 * MB];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int m = 0; m < MB; ++m) hv[i * MB + m] = (_Float16)d[m][4 * g + i];
#pragma unroll
        for (int q = 0; q < MB / 2; ++q) {
          u4 v;
#pragma unroll
          for (int w = 0; w < 4; ++w)
            v[w] = (uint32_t)__builtin_bit_cast(uint16_t, hv[8 * q + 2 * w]) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, hv[8 * q + 2 * w + 1]) << 16);
          *reinterpret_cast<u4*>(dst + 16u * q) = v;
        }
      }
    }
  }
  __syncthreads();

  const h2 e0 = {(_Float16)1.0f, (_Float16)0.0f}, e1 = {(_Float16)0.0f, (_Float16)1.0f};
  auto step = [&](int i, const St& st, St& nxt) {
    load_stage(i + D - 1, nxt);
    float acc[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = 0.f;
#pragma unroll
    for (int g = 0; g < 2 * PP; ++g) {
      float part[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) part[m] = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
          const uint32_t w = st.c[2 * g + t][dw];
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const uint32_t sg = 32u * g + 16u * t + 4u * dw + bb;
            const uint32_t addr = __builtin_amdgcn_ubfe(w, 8 * bb, 8) * EB + (sg / SB) * (SB * BS);
            const char* const src = lds + addr + BS * (sg % SB);
            if constexpr (MB == 2) {
              const h2 v = as_h2(*reinterpret_cast<const uint32_t*>(src));
              part[0] = dot2(v, e0, part[0]);
              part[1] = dot2(v, e1, part[1]);
            } else {
              const u2 v = *reinterpret_cast<const u2*>(src);
              part[0] = dot2(as_h2(v.x), e0, part[0]);
              part[1] = dot2(as_h2(v.x), e1, part[1]);
              part[2] = dot2(as_h2(v.y), e0, part[2]);
              part[3] = dot2(as_h2(v.y), e1, part[3]);
            }
          }
        }
      }
      const float sc = h2f((uint16_t)(st.s[g / 2] >> (16 * (g % 2))));
#pragma unroll
      for (int m = 0; m < MB; ++m) acc[m] = fmaf(sc, part[m], acc[m]);
    }
    const uint32_t row = (uint32_t)(rb0 + i * RS) * 64u + lane;
    if (row < (uint32_t)N) {
#pragma unroll
      for (int m = 0; m < MB; ++m) {
        if (m0 + m >= M) break;
        if (KP == 1)
          a.y[(size_t)(m0 + m) * N + row] = f2h(acc[m]);
        else
          a.ws[((size_t)kp * M + m0 + m) * N + row] = acc[m];
      }
    }
  };
  for (int i = 0; i < cnt; i += D) {
#pragma unroll
    for (int k = 0; k < D; ++k)
      if (i + k < cnt) step(i + k, ring[k], ring[(k + D - 1) % D]);
  }
}

// y[i] = fp16(sum over k < KS of ws[k * MN + i]).  A workgroup takes 64
// outputs; wave j adds parts j, j + 8, j + 16, ... (loads issued 8 at a time,
// each a 256-byte row), and wave 0 adds the 8 wave sums in order: a fixed
// order for every output, so the result is deterministic.
// General codebook kernel (CodeGEMM notes, key design 3: one kernel for any
// number of codebooks m, vector length v, code bits b and group size g):
// NCB additive codebooks of 256 centroids of V dims (V = 4, 8, 16), 8-bit
// codes, one scale per g k (g = 32, 64, 128), and at most 2 code bits per
// weight (NCB * 256 / V <= 64), so the Psumbook rows of a 256-k chunk -- row
// i * S + s for codebook i and segment s, S = 256 / V -- fit the same
// 64-row table as the single-codebook kernels.
//   w[n, V j + t] = s[n, (V j + t) / g] * sum_i C_i[code_i[n, j]][t]
//   P_i[j][c]    = sum_t C_i[c][t] * x[m, V j + t]
//   y[m, n]      = sum_groups s[n, group] * sum_{j in group} sum_i P_i[j][code_i[n, j]]
// Codes are NCB planes, each an [N, K/V] uint8 matrix in the 64-row layout.
// A workgroup of 4 waves owns 4 row blocks and a K range.  Per chunk:
// LDS barrier, the build on the matrix cores (v_mfma_f32_32x32x8_f16, A =
// codebook rows with their dims in 8-wide steps, zero-padded for V = 4, B =
// activation segments; tasks (codebook, centroid block, segment block) dealt
// to the waves in turn), LDS barrier, then each lane looks up its own row's
// codes, pairs of segments summed by one v_dot2, a group partial scaled once.
// The next chunk's codes, scales and activation segments are in flight
// meanwhile.  K parts (KS > 1) go through the workspace and the reduce kernel.
template <int V, int NCB>
__global__ void __launch_bounds__(256) gemv_codebook_gen_kernel(CodebookGenArgs a) {
  constexpr int S = 256 / V;           // segments per chunk and codebook
  constexpr int NT = S / 16;           // 16-code tiles per chunk and plane
  constexpr int SB = (S + 31) / 32;    // 32-segment blocks
  constexpr int NST = V <= 8 ? 1 : 2;  // 8-dim MFMA steps
  constexpr int T = NCB * 8 * SB;      // build tasks per chunk
  constexpr int TW = (T + 3) / 4;      // tasks per wave
  static_assert(NCB * S <= 64, "a chunk's Psumbook rows fit the table");
  __shared__ __attribute__((aligned(16))) uint32_t lsm[PSUM_BYTES / 4];
  char* const lds = reinterpret_cast<char*>(lsm);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = a.M, N = a.N, K = a.K, GS = a.group;
  const int HN = K / 256;  // chunks
  const int NB = (N + 63) / 64;
  const int CPR = K / V / 16;  // code tiles per row block and plane
  const uint32_t PLANE = (uint32_t)NB * CPR * 1024u;
  const int GPR = K / GS;   // scale groups per row
  const int NG = 256 / GS;  // scale groups per chunk
  const int m = blockIdx.z;
  const int ks = blockIdx.y, KS = gridDim.y;
  const int h0 = (HN * ks) / KS, h1 = (HN * (ks + 1)) / KS;
  const int rb = blockIdx.x * 4 + wave;  // this wave's 64-row block
  const uint32_t row = (uint32_t)rb * 64u + lane;
  const bool rv = rb < NB && row < (uint32_t)N;
  const int li = lane & 31, hi = lane >> 5;

  const rsrc_t rc = make_rsrc(a.codes, PLANE * NCB);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * GPR * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);

  // A operands, kept for the whole kernel: task u = wave + 4 j is codebook
  // u / (8 SB), centroid block (u / SB) % 8, segment block u % SB; lane l
  // holds centroid 32 cb + l % 32, dims 8 step + 4 (l / 32) .. + 3
  h4v ca[TW][NST];
  {
    const rsrc_t rcb = make_rsrc(a.codebooks, NCB * 256u * V * 2u);
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int u = wave + 4 * j, ci = u / (8 * SB), cb = (u / SB) % 8;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int d0 = 8 * st + 4 * hi;
        const bool ok = u < T && d0 < V;
        ca[j][st] = __builtin_bit_cast(
            h4v, __builtin_amdgcn_raw_buffer_load_b64(rcb, ok ? (uint32_t)(((ci * 256 + 32 * cb + li) * V + d0) * 2) : OOB,
                                                      0, 0));
      }
    }
  }
  struct St {
    u4 c[NCB * NT];  // this lane's row's codes of the chunk, per plane
    uint16_t s[8];   // the chunk's scales of this row
    u2 xb[TW][NST];  // B operands of this wave's tasks
  };
  const uint32_t vcode = rb < NB ? 16u * lane : OOB;
  const uint32_t vscale = rv ? row * (uint32_t)GPR * 2u : OOB;
  auto load_stage = [&](int h, St& st) {
    const uint32_t hc = (uint32_t)min(h, h1 - 1);  // (past the range: a harmless re-read)
#pragma unroll
    for (int i = 0; i < NCB; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t so = __builtin_amdgcn_readfirstlane(
            (uint32_t)i * PLANE + ((uint32_t)min(rb, NB - 1) * CPR + hc * NT + t) * 1024u);
        st.c[i * NT + t] = bload16<CPOL_NT>(rc, vcode, so);
      }
#pragma unroll
    for (int gg = 0; gg < 8; ++gg)
      if (gg < NG) st.s[gg] = bload2(rs, vscale, (hc * NG + gg) * 2u);
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int u = wave + 4 * j, seg = 32 * (u % SB) + li;
#pragma unroll
      for (int st2 = 0; st2 < NST; ++st2) {
        const int d0 = 8 * st2 + 4 * hi;
        const bool ok = u < T && seg < S && d0 < V;
        st.xb[j][st2] = __builtin_bit_cast(
            u2, __builtin_amdgcn_raw_buffer_load_b64(
                    rx, ok ? ((uint32_t)m * K + 256u * hc + (uint32_t)(V * seg + d0)) * 2u : OOB, 0, 0));
      }
    }
  };

  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  float acc = 0.f;
  auto step = [&](int h, const St& st, St& nxt) {
    load_stage(h + 1, nxt);
    lds_barrier();  // every wave is done reading the previous chunk's P
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int u = wave + 4 * j;
      if (u < T) {  // (wave-uniform)
        const int ci = u / (8 * SB), cb = (u / SB) % 8, seg = 32 * (u % SB) + li;
        f16v d = f16v{};
#pragma unroll
        for (int st2 = 0; st2 < NST; ++st2)
          d = __builtin_amdgcn_mfma_f32_32x32x8f16(ca[j][st2], __builtin_bit_cast(h4v, st.xb[j][st2]), d, 0, 0, 0);
        // lane l, register 4 g + r: P_ci[seg][32 cb + 8 g + 4 (l / 32) + r]
        if (seg < S) {
          char* const base = lds + (uint32_t)(ci * S + seg) * PSTRIDE + 2u * (32u * cb + 4u * hi);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const h4v hv = {(_Float16)d[4 * g], (_Float16)d[4 * g + 1], (_Float16)d[4 * g + 2], (_Float16)d[4 * g + 3]};
            *reinterpret_cast<u2*>(base + 16u * g) = __builtin_bit_cast(u2, hv);
          }
        }
      }
    }
    lds_barrier();  // P of this chunk complete
    // lookups: segments in pairs (a group holds at least 2 segments, an even
    // number), the group partial scaled once
    float part = 0.f;
#pragma unroll
    for (int sp = 0; sp < S; sp += 2) {
#pragma unroll
      for (int i = 0; i < NCB; ++i) {
        h2 pv;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int sg = sp + e;
          const uint32_t w = st.c[i * NT + sg / 16][(sg % 16) / 4];
          const uint32_t code2 = __builtin_amdgcn_ubfe(w, 8 * (sg % 4), 8) << 1;
          pv[e] = *reinterpret_cast<const _Float16*>(lds + code2 + PSTRIDE * (uint32_t)(i * S + sg));
        }
        part = dot2(pv, ones, part);
      }
      if (((sp + 2) * V) % GS == 0) {  // (wave-uniform) end of a scale group
        const int gi = (sp * V) / GS;
        uint16_t sc = st.s[0];
#pragma unroll
        for (int gg = 1; gg < 8; ++gg) sc = gg == gi ? st.s[gg] : sc;  // (no dynamic register index)
        acc = fmaf(h2f(sc), part, acc);
        part = 0.f;
      }
    }
  };
  St ring[2];
  load_stage(h0, ring[0]);
  for (int h = h0; h < h1; h += 2) {  // two chunks per iteration so the stages are named statically
    step(h, ring[0], ring[1]);
    if (h + 1 < h1) step(h + 1, ring[1], ring[0]);
  }
  if (!rv) return;
  if (KS == 1)
    a.y[(size_t)m * N + row] = f2h(acc);
  else  // K split: this range's partial sum, added up by the reduce kernel
    a.ws[((size_t)ks * M + m) * N + row] = acc;
}

// Stationary form of the general kernel: a workgroup of WK waves owns one
// 256-k chunk h and one batch row, builds the chunk's Psumbooks once, and
// streams row blocks through them (wave w of row slice r takes row blocks
// r WK + w + i R WK, the next one in flight) with no barrier after the build; each row's partial sum
// for the chunk goes to the workspace, and the reduce kernel adds the chunks
// in a fixed order.  Grid: R x K/256 x M workgroups.
template <int V, int NCB>
__global__ void __launch_bounds__(256) gemv_codebook_gen_stat_kernel(CodebookGenArgs a, int R) {
  constexpr int S = 256 / V;
  constexpr int NT = S / 16;
  constexpr int SB = (S + 31) / 32;
  constexpr int NST = V <= 8 ? 1 : 2;
  constexpr int T = NCB * 8 * SB;
  static_assert(NCB * S <= 64, "a chunk's Psumbook rows fit the table");
  __shared__ __attribute__((aligned(16))) uint32_t lsm[PSUM_BYTES / 4];
  char* const lds = reinterpret_cast<char*>(lsm);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int WK = blockDim.x >> 6;
  const int M = a.M, N = a.N, K = a.K, GS = a.group;
  const int NB = (N + 63) / 64;
  const int CPR = K / V / 16;
  const uint32_t PLANE = (uint32_t)NB * CPR * 1024u;
  const int GPR = K / GS, NG = 256 / GS;
  const int r = blockIdx.x, h = blockIdx.y, m = blockIdx.z;
  const int li = lane & 31, hi = lane >> 5;
  const rsrc_t rc = make_rsrc(a.codes, PLANE * NCB);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * GPR * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);

  // the row blocks this wave streams, each with its codes and scales
  struct St {
    u4 c[NCB * NT];
    uint16_t s[8];
  };
  auto load_rows = [&](int rb, St& st) {
    const bool bv = rb < NB;  // (past the last block: zeros, never used)
    const uint32_t vcode = bv ? 16u * lane : OOB;
    const uint32_t row = (uint32_t)rb * 64u + lane;
    const uint32_t vscale = bv && row < (uint32_t)N ? row * (uint32_t)GPR * 2u : OOB;
#pragma unroll
    for (int i = 0; i < NCB; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t so = __builtin_amdgcn_readfirstlane(
            (uint32_t)i * PLANE + ((uint32_t)min(rb, NB - 1) * CPR + (uint32_t)h * NT + t) * 1024u);
        st.c[i * NT + t] = bload16<CPOL_NT>(rc, vcode, so);
      }
#pragma unroll
    for (int gg = 0; gg < 8; ++gg)
      if (gg < NG) st.s[gg] = bload2(rs, vscale, ((uint32_t)h * NG + gg) * 2u);
  };
  const int step_rb = R * WK;
  int rb = r * WK + wave;
  St ring[2];
  // the activation segments and codebook rows of the build are issued first:
  // a wave's loads return in order
  {
    const rsrc_t rcb = make_rsrc(a.codebooks, NCB * 256u * V * 2u);
    for (int u = wave; u < T; u += WK) {  // (wave-uniform)
      const int ci = u / (8 * SB), cb = (u / SB) % 8, seg = 32 * (u % SB) + li;
      f16v d = f16v{};
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int d0 = 8 * st + 4 * hi;
        const h4v av = __builtin_bit_cast(
            h4v, __builtin_amdgcn_raw_buffer_load_b64(
                     rcb, d0 < V ? (uint32_t)(((ci * 256 + 32 * cb + li) * V + d0) * 2) : OOB, 0, 0));
        const h4v bv = __builtin_bit_cast(
            h4v, __builtin_amdgcn_raw_buffer_load_b64(
                     rx, seg < S && d0 < V ? ((uint32_t)m * K + 256u * h + (uint32_t)(V * seg + d0)) * 2u : OOB, 0,
                     0));
        d = __builtin_amdgcn_mfma_f32_32x32x8f16(av, bv, d, 0, 0, 0);
      }
      if (seg < S) {
        char* const base = lds + (uint32_t)(ci * S + seg) * PSTRIDE + 2u * (32u * cb + 4u * hi);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const h4v hv = {(_Float16)d[4 * g], (_Float16)d[4 * g + 1], (_Float16)d[4 * g + 2], (_Float16)d[4 * g + 3]};
          *reinterpret_cast<u2*>(base + 16u * g) = __builtin_bit_cast(u2, hv);
        }
      }
    }
  }
  load_rows(rb, ring[0]);
  __syncthreads();  // the Psumbooks are complete

  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  auto lookups = [&](int rbk, const St& st, St& nxt) {
    load_rows(rbk + step_rb, nxt);
    float acc = 0.f, part = 0.f;
#pragma unroll
    for (int sp = 0; sp < S; sp += 2) {
#pragma unroll
      for (int i = 0; i < NCB; ++i) {
        h2 pv;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int sg = sp + e;
          const uint32_t w = st.c[i * NT + sg / 16][(sg % 16) / 4];
          const uint32_t code2 = __builtin_amdgcn_ubfe(w, 8 * (sg % 4), 8) << 1;
          pv[e] = *reinterpret_cast<const _Float16*>(lds + code2 + PSTRIDE * (uint32_t)(i * S + sg));
        }
        part = dot2(pv, ones, part);
      }
      if (((sp + 2) * V) % GS == 0) {  // (wave-uniform) end of a scale group
        const int gi = (sp * V) / GS;
        uint16_t sc = st.s[0];
#pragma unroll
        for (int gg = 1; gg < 8; ++gg) sc = gg == gi ? st.s[gg] : sc;  // (no dynamic register index)
        acc = fmaf(h2f(sc), part, acc);
        part = 0.f;
      }
    }
    const uint32_t row = (uint32_t)rbk * 64u + lane;
    if (row < (uint32_t)N) a.ws[((size_t)h * M + m) * N + row] = acc;
  };
  for (; rb < NB; rb += 2 * step_rb) {  // two row blocks per iteration so the stages are named statically
    lookups(rb, ring[0], ring[1]);
    if (rb + step_rb < NB) lookups(rb + step_rb, ring[1], ring[0]);
  }
}

__global__ void __launch_bounds__(512) codebook_reduce_kernel(const float* __restrict__ ws, uint16_t* __restrict__ y,
                                                              int MN, int KS) {
  __shared__ float part[8][64];
  const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + lane;
  float sum = 0.f;
  if (i < MN) {
    int k = j;
    for (; k + 56 < KS; k += 64) {
      float v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = __builtin_nontemporal_load(&ws[(size_t)(k + 8 * t) * MN + i]);
#pragma unroll
      for (int t = 0; t < 8; ++t) sum += v[t];
    }
    for (; k < KS; k += 8) sum += __builtin_nontemporal_load(&ws[(size_t)k * MN + i]);
  }
  part[j][lane] = sum;
  __syncthreads();
  if (j == 0 && i < MN) {
    float t = part[0][lane];
#pragma unroll
    for (int w = 1; w < 8; ++w) t += part[w][lane];
    y[i] = f2h(t);
  }
}

template <int NSB>
void* seq_kernel_ptr(bool sal) {
  return sal ? reinterpret_cast<void*>(&gemv_codebook_seq_kernel<NSB, true>)
             : reinterpret_cast<void*>(&gemv_codebook_seq_kernel<NSB, false>);
}

template <int MB, int PP>
void* statb_kernel_ptr(bool sal) {
  return sal ? reinterpret_cast<void*>(&gemv_codebook_statb_kernel<MB, PP, true>)
             : reinterpret_cast<void*>(&gemv_codebook_statb_kernel<MB, PP, false>);
}

template <int PP>
void* stat_kernel_ptr(bool sal) {
  return sal ? reinterpret_cast<void*>(&gemv_codebook_stat_kernel<PP, true>)
             : reinterpret_cast<void*>(&gemv_codebook_stat_kernel<PP, false>);
}

}  // namespace

// K parts a launch writes partial sums for (1: none, y directly)
static int codebook_parts(const CodebookCfg& c, int K) { return c.pp > 0 ? K / (256 * c.pp) : c.ks; }

// Workspace: parts x M x N fp32 partial sums; scratch, no initial contents.
size_t codebook_ws_bytes(const CodebookCfg& c, int M, int N, int K) {
  const int parts = codebook_parts(c, K);
  return parts > 1 ? (size_t)parts * M * N * 4 : 0;
}

// Fitted to sweeps on MI355X (8B- and 70B-shaped layers, M = 1, 2 and 4).
//  * The stationary kernel wins where there are many rows to stream through
//    each Psumbook: N >= 10240 at M = 1 (two pairs per part once K >= 8192,
//    about 256 workgroups), and at M >= 2 any layer of 32M weights or more.
//  * At M >= 2 its Psumbook entries hold a block of batch rows (2 at M = 2
//    or N < 8192, else 4), so one lookup serves the whole block: one pair per
//    part, 8 waves with 4-row entries (4 with 2-row ones), about 256
//    workgroups in all.  70B gate+up at M = 4: 98 -> 52 us.
//  * Elsewhere (fewer rows, or K long against N) the sequential kernel, with
//    K split in whole pairs until the grid holds about 384 workgroups.
CodebookCfg pick_codebook(int M, int N, int K) {
  CodebookCfg c;
  c.wk = 4;
  c.mb = 1;
  const long NB = (N + 63) / 64;
  const long HN = K / 256;
  const bool stat = M == 1 ? N >= 10240 : (long)N * K >= (32L << 20);
  if (stat && M >= 2) {
    c.mb = M == 2 || N < 8192 ? 2 : 4;
    c.wk = c.mb == 4 ? 8 : 4;
    c.pp = 1;
    c.ks = 1;
    const long rg = (NB + c.wk - 1) / c.wk;
    const long units = HN * ((M + c.mb - 1) / c.mb);  // workgroups per row slice
    c.r = (int)std::max(1L, std::min(rg, (256 + units / 2) / units));
  } else if (stat) {
    c.pp = K >= 8192 && HN % 2 == 0 ? 2 : 1;
    c.ks = 1;
    const long rg = (NB + c.wk - 1) / c.wk;
    const long KP = HN / c.pp;
    c.r = (int)std::max(1L, std::min(rg, (256 + KP - 1) / KP));
  } else {
    const long rg = (NB + c.wk - 1) / c.wk;
    c.pp = 0;
    c.r = 0;
    c.ks = 1;
    while (c.ks * 2 <= HN && rg * M * c.ks < 384) c.ks *= 2;
  }
  return c;
}

CodebookCfg codebook_fallback() {
  CodebookCfg c;
  c.wk = 4;
  c.mb = 1;
  c.pp = 0;
  c.r = 0;
  c.ks = 1;
  return c;
}

hipError_t launch_gemv_codebook(const CodebookArgs& a, const CodebookCfg& c, hipStream_t s) {
  if (c.wk != 1 && c.wk != 2 && c.wk != 4 && c.wk != 8 && c.wk != 16) return hipErrorInvalidValue;
  const int parts = codebook_parts(c, a.K);
  const bool sal = reinterpret_cast<uintptr_t>(a.scales) % 4 == 0;
  if (c.pp > 0) {
    // four pairs, or two pairs of 2-row entries, or one pair of 4-row entries:
    // about 133 KB of Psumbook, one workgroup per CU, at most 8 waves
    const bool big = c.pp * c.mb >= 4 || c.mb > 1;  // (the batched kernels: at most 8 waves)
    if ((c.pp != 1 && c.pp != 2 && c.pp != 4) || (c.mb != 1 && c.mb != 2 && c.mb != 4) || c.pp * c.mb > 4 ||
        (big && c.wk > 8) || (a.K / 256) % c.pp || c.r < 1 || c.r > (1 << 20))
      return hipErrorInvalidValue;
    if (parts > 1 && !a.ws) return hipErrorInvalidValue;
    const long units = (long)c.r * parts;
    const long blocks = (units + 7) / 8 * 8 * ((a.M + c.mb - 1) / c.mb);
    if (blocks >= (1L << 31)) return hipErrorInvalidValue;
    void* const kern = c.mb == 4   ? statb_kernel_ptr<4, 1>(sal)
                       : c.mb == 2 ? (c.pp == 1 ? statb_kernel_ptr<2, 1>(sal) : statb_kernel_ptr<2, 2>(sal))
                       : c.pp == 1 ? stat_kernel_ptr<1>(sal)
                       : c.pp == 2 ? stat_kernel_ptr<2>(sal)
                                   : stat_kernel_ptr<4>(sal);
    int r = c.r;
    void* args[] = {const_cast<CodebookArgs*>(&a), &r};
    hipError_t e = hipLaunchKernel(kern, dim3((unsigned)blocks), dim3(64 * c.wk), args, 0, s);
    if (e != hipSuccess) return e;
  } else {
    if (c.ks < 1 || c.ks > a.K / 256 || (c.ks > 1 && !a.ws)) return hipErrorInvalidValue;
    const int NB = (a.N + 63) / 64;
    const dim3 grid((unsigned)((NB + c.wk - 1) / c.wk), c.ks, a.M);
    void* const kern = c.wk == 1 ? seq_kernel_ptr<2>(sal) : seq_kernel_ptr<1>(sal);
    void* args[] = {const_cast<CodebookArgs*>(&a)};
    hipError_t e = hipLaunchKernel(kern, grid, dim3(64 * c.wk), args, 0, s);
    if (e != hipSuccess) return e;
  }
  if (parts > 1) {
    const int MN = a.M * a.N;
    hipLaunchKernelGGL(codebook_reduce_kernel, dim3((MN + 63) / 64), dim3(512), 0, s, a.ws, a.y, MN, parts);
  }
  return hipGetLastError();
}

// General codebook kernel dispatch (sweeps of the 8B layers at M = 1 for
// (m, v, g) = (1, 4, 128), (3, 16, 32), (2, 8, 64)): the stationary form
// with 4 waves up to K = 8192 (returned as -4), else the sequential form
// with K parts such that the grid has about 512 workgroups (each walks at
// least one 256-k chunk).
int codebook_gen_ks(int M, int N, int K) {
  if (K <= 8192 && K >= 512) return -4;
  const int wgs = ((N + 63) / 64 + 3) / 4 * M;
  int ks = (512 + wgs - 1) / wgs;
  if (ks > K / 256) ks = K / 256;
  return ks < 1 ? 1 : ks;
}

size_t codebook_gen_ws_bytes(int M, int N, int K) {
  // room for the stationary form's one partial per 256-k chunk (the most parts)
  return K / 256 > 1 ? (size_t)(K / 256) * M * N * 4 : 0;
}

template <int V, int NCB>
void* gen_kernel_ptr() {
  return reinterpret_cast<void*>(&gemv_codebook_gen_kernel<V, NCB>);
}

template <int V, int NCB>
void* gen_stat_kernel_ptr() {
  return reinterpret_cast<void*>(&gemv_codebook_gen_stat_kernel<V, NCB>);
}

// stationary form: R row slices per chunk, about 256 workgroups
int codebook_gen_stat_r(int M, int N, int K, int wk) {
  const int rmax = ((N + 63) / 64 + wk - 1) / wk;
  int r = (256 + (K / 256) * M - 1) / ((K / 256) * M);
  return r < 1 ? 1 : (r > rmax ? rmax : r);
}

hipError_t launch_gemv_codebook_gen(const CodebookGenArgs& a, int ks, hipStream_t s) {
  void* kern = nullptr;
  const bool stat = ks < 0;  // stationary: one K part per 256-k chunk
  switch (a.v * 10 + a.ncb) {
    case 41: kern = stat ? gen_stat_kernel_ptr<4, 1>() : gen_kernel_ptr<4, 1>(); break;
    case 81: kern = stat ? gen_stat_kernel_ptr<8, 1>() : gen_kernel_ptr<8, 1>(); break;
    case 82: kern = stat ? gen_stat_kernel_ptr<8, 2>() : gen_kernel_ptr<8, 2>(); break;
    case 161: kern = stat ? gen_stat_kernel_ptr<16, 1>() : gen_kernel_ptr<16, 1>(); break;
    case 162: kern = stat ? gen_stat_kernel_ptr<16, 2>() : gen_kernel_ptr<16, 2>(); break;
    case 163: kern = stat ? gen_stat_kernel_ptr<16, 3>() : gen_kernel_ptr<16, 3>(); break;
    case 164: kern = stat ? gen_stat_kernel_ptr<16, 4>() : gen_kernel_ptr<16, 4>(); break;
    default: return hipErrorInvalidValue;
  }
  if (stat) {
    if (!a.ws) return hipErrorInvalidValue;
    const int wk = -ks, HN = a.K / 256;
    if (wk < 1 || wk > 4) return hipErrorInvalidValue;
    int R = codebook_gen_stat_r(a.M, a.N, a.K, wk);
    void* args[] = {const_cast<CodebookGenArgs*>(&a), &R};
    hipError_t e = hipLaunchKernel(kern, dim3(R, HN, a.M), dim3(64 * wk), args, 0, s);
    if (e != hipSuccess) return e;
    const int MN = a.M * a.N;
    hipLaunchKernelGGL(codebook_reduce_kernel, dim3((MN + 63) / 64), dim3(512), 0, s, a.ws, a.y, MN, HN);
    return hipGetLastError();
  }
  if (ks < 1 || ks > a.K / 256 || (ks > 1 && !a.ws)) return hipErrorInvalidValue;
  const int NB = (a.N + 63) / 64;
  const dim3 grid((unsigned)((NB + 3) / 4), ks, a.M);
  void* args[] = {const_cast<CodebookGenArgs*>(&a)};
  hipError_t e = hipLaunchKernel(kern, grid, dim3(256), args, 0, s);
  if (e != hipSuccess) return e;
  if (ks > 1) {
    const int MN = a.M * a.N;
    hipLaunchKernelGGL(codebook_reduce_kernel, dim3((MN + 63) / 64), dim3(512), 0, s, a.ws, a.y, MN, ks);
  }
  return hipGetLastError();
}

}  // namespace qg
