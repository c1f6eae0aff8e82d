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
//    its own row's 16 codes.  A "quad" of 4 quant groups (128 segments, 512 k)
//    is 8 consecutive tiles of a row block, 8 KB contiguous.
//  * Psumbook of a quad in LDS, segment-major: fp16 P[s][c] at byte
//    512 s + 2 c (64 KB).  All lanes of a wave look up the same segment s at
//    once, so s is the instruction's immediate offset and the lane address is
//    2 * code; the bank follows the (random) code, not the segment.  Two
//    lookups are summed into the fp32 partial by one v_dot2 against (1, 1).
//    Each lane owns one weight row, so no cross-lane reduction is needed.
//  * Build on the matrix cores: one v_mfma_f32_32x32x8_f16 gives P for 32
//    segments x 32 centroids (A = activation segments, B = codebook rows, the
//    v = 4 dims padded to 8 with zeros); 32 of them per quad, spread over the
//    waves of the workgroup.
//  * Work split: a workgroup holds WK waves, one 64-row block each, and a K
//    range of whole quads; one build serves 64 * WK rows.  The K ranges of a
//    row block are reduced in a fixed order by the last of their workgroups
//    to finish (a counter per row block in the caller's workspace), so the
//    result is deterministic.  Batch rows are grid z.
//  * Per quad: build / LDS barrier / lookups, with the next quad's codes,
//    scales and activation segments in flight meanwhile.  The barriers wait
//    for LDS traffic only, so those prefetches stay outstanding across them.
#include "common.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

constexpr uint32_t PSUM_BYTES = 128u * 256u * 2u;  // 128 segments x 256 centroids x fp16
constexpr uint32_t CB_BYTES = 256u * 4u * 2u;      // the codebook, staged

typedef _Float16 h4v __attribute__((ext_vector_type(4)));

// SAL: the scales base is 8-byte aligned, so a quad's 4 scales of a row are
// one load (K is a multiple of 512, so every row's quad starts 8-aligned too).
template <bool SAL>
__global__ void __launch_bounds__(1024) gemv_codebook_kernel(CodebookArgs a) {
  // LDS: [Psumbook 64 KB][codebook 2 KB][flag]
  extern __shared__ __attribute__((aligned(16))) uint32_t lsm[];
  char* const lds = reinterpret_cast<char*>(lsm);
  uint32_t* const flag = reinterpret_cast<uint32_t*>(lds + PSUM_BYTES + CB_BYTES);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int WK = blockDim.x >> 6;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / 128;   // quant groups
  const int QN = K / 512;  // quads
  const int NCB = K / 64;  // 16-code tiles per row block
  const int NB = (N + 63) / 64;
  const int m = blockIdx.z;
  const int ks = blockIdx.y, KS = gridDim.y;
  const int q0 = (QN * ks) / KS, q1 = (QN * (ks + 1)) / KS;
  const int rb = blockIdx.x * WK + wave;  // this wave's 64-row block
  const uint32_t row = (uint32_t)rb * 64u + lane;
  const bool rv = rb < NB && row < (uint32_t)N;

  const rsrc_t rc = make_rsrc(a.codes, (uint32_t)NB * NCB * 1024u);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * G * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);

  struct St {
    u4 c[8];        // 8 tiles x 16 codes of this lane's row
    uint16_t s[4];  // the quad's 4 group scales of this row
  };
  // Loads are unconditional, with every choice in the offsets: a wave past
  // the last row block reads zero codes, a row past N zero scales.  The
  // prefetch past the K range re-reads the range's last quad (never used),
  // so that the quad index only ever moves the wave-uniform offsets.
  const uint32_t vcode = rb < NB ? 16u * lane : OOB;
  const uint32_t vscale = rv ? row * (uint32_t)G * 2u : OOB;
  auto load_stage = [&](int q, St& st) {
    const uint32_t qc = (uint32_t)min(q, q1 - 1);
    const uint32_t sw = __builtin_amdgcn_readfirstlane(((uint32_t)min(rb, NB - 1) * NCB + 8u * qc) * 1024u);
#pragma unroll
    for (int i = 0; i < 8; ++i) st.c[i] = bload16<CPOL_NT>(rc, vcode + 1024u * i, sw);
    if constexpr (SAL) {
      const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rs, vscale, 8u * qc, 0));
#pragma unroll
      for (int g = 0; g < 4; ++g) st.s[g] = (uint16_t)(v[g / 2] >> (16 * (g % 2)));
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g) st.s[g] = bload2(rs, vscale, 8u * qc + 2u * g);
    }
  };

  // build assignment: wave w computes blocks p = w, w + WK, ... (p < 32) of 32
  // segments (sb = p % 4) x 32 centroids (cb = p / 4); WK % 4 == 0 keeps sb
  // fixed per wave, so each wave needs one activation operand per quad
  const int sbw = wave & 3;
  const int li = lane & 31;
  const bool klo = lane < 32;  // lanes holding dims 0..3 (the others: the zero padding)
  const uint32_t vx = klo ? ((uint32_t)m * K + 4u * (32u * sbw + li)) * 2u : OOB;
  auto load_xseg = [&](int q) -> u2 {  // segment 32 sb + l % 32 of quad q: 4 halves
    const uint32_t qc = (uint32_t)min(q, q1 - 1);
    return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rx, vx, 1024u * qc, 0));
  };

  St ring[2];
  load_stage(q0, ring[0]);
  u2 xseg = load_xseg(q0);

  // codebook into LDS once (read by the build as B operands)
  {
    const rsrc_t rcb = make_rsrc(a.codebook, CB_BYTES);
    for (int i = threadIdx.x; i < 512; i += blockDim.x) lsm[(PSUM_BYTES / 4) + i] = bload4(rcb, 4u * i);
  }
  const u2* cbv = reinterpret_cast<const u2*>(lds + PSUM_BYTES);
  _Float16* const P16 = reinterpret_cast<_Float16*>(lds);
  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  float acc = 0.f;

  auto step = [&](int q, const St& st, St& nxt) {
    load_stage(q + 1, nxt);  // next quad (past the range: a harmless re-read)
    const u2 xnext = load_xseg(q + 1);
    lds_barrier();  // every wave is done reading the previous quad's P (and the codebook is staged)
    for (int p = wave; p < 32; p += WK) {
      const int cb = p >> 2;
      const u2 cv = cbv[32 * cb + li];
      const u2 cc = {klo ? cv.x : 0u, klo ? cv.y : 0u};
      const f16v d = __builtin_amdgcn_mfma_f32_32x32x8f16(__builtin_bit_cast(h4v, xseg), __builtin_bit_cast(h4v, cc),
                                                          f16v{}, 0, 0, 0);
      // lane l, register r: P[32 sb + 8 (r / 4) + 4 (l / 32) + r % 4][32 cb + l % 32]
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int s = 32 * sbw + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        P16[s * 256 + 32 * cb + li] = (_Float16)d[r];
      }
    }
    xseg = xnext;
    lds_barrier();  // P of this quad complete
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float part = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // tile 2g + h: segments 32g + 16h + 0..15
#pragma unroll
        for (int d = 0; d < 4; ++d) {  // word d: segments 32g + 16h + 4d + 0..3
          const uint32_t w = st.c[2 * g + h][d];
          const uint32_t s0 = 32u * g + 16u * h + 4u * d;
          h2 pa, pb;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const uint32_t code2 = ((w >> (8 * b)) & 0xFFu) << 1;
            const _Float16 v = *reinterpret_cast<const _Float16*>(lds + code2 + 512u * (s0 + b));
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
  // two quads per iteration so the stage buffers are named statically
  for (int q = q0; q < q1; q += 2) {
    step(q, ring[0], ring[1]);
    if (q + 1 < q1) step(q + 1, ring[1], ring[0]);
  }

  if (KS == 1) {
    if (rv) a.y[(size_t)m * N + row] = f2h(acc);
    return;
  }
  // K split: partial sums to the workspace; the last workgroup of the row
  // block adds them in K order
  if (rv) a.ws[((size_t)ks * M + m) * N + row] = acc;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* cnt = a.cnt + (size_t)m * gridDim.x + blockIdx.x;
    const uint32_t old = atomicAdd(cnt, 1u);
    const bool last = old == (uint32_t)KS - 1u;
    if (last) *cnt = 0u;  // ready for the next call
    *flag = last;
  }
  __syncthreads();
  if (*flag) {
    __threadfence();
    if (rv) {
      float sum = 0.f;
      for (int k = 0; k < KS; ++k) sum += __builtin_nontemporal_load(&a.ws[((size_t)k * M + m) * N + row]);
      a.y[(size_t)m * N + row] = f2h(sum);
    }
  }
}

}  // namespace

// Workspace: KS x M x N fp32 partial sums from the start, and a fixed area of
// CB_COUNTERS counters (one per batch row and row block) at the very end of
// the caller's buffer, so that shapes sharing one workspace never write their
// partial sums over each other's counters.  The counters must be zero before
// first use; every call leaves them zero.
size_t codebook_ws_bytes(const CodebookCfg& c, int M, int N) {
  if (c.ks <= 1) return 0;
  return (size_t)c.ks * M * N * 4 + CB_COUNTERS * 4;
}

size_t codebook_row_blocks(const CodebookCfg& c, int N) {
  const int NB = (N + 63) / 64;
  return (NB + c.wk - 1) / c.wk;
}

// Measured on MI355X (70B-class layers, M = 1 and 4): the best launches fill
// the 256 CUs with about one workgroup each.  Take the fewest waves per
// workgroup (the cheapest barriers) whose row blocks x batch rows fit in 256
// workgroups, then split K (whole quads) while the grid still fits.
CodebookCfg pick_codebook(int M, int N, int K) {
  CodebookCfg c;
  c.wk = 16;
  for (int wk = 4; wk <= 16; wk *= 2) {
    c.wk = wk;
    if ((long)codebook_row_blocks(c, N) * M <= 256) break;
  }
  const long wgs = (long)codebook_row_blocks(c, N) * M;
  const int QN = K / 512;
  c.ks = 1;
  while (c.ks * 2 <= QN && wgs * c.ks * 2 <= 256) c.ks *= 2;
  return c;
}

hipError_t launch_gemv_codebook(const CodebookArgs& a, const CodebookCfg& c, hipStream_t s) {
  // the Psumbook build gives each wave a fixed segment block: wk % 4 == 0
  if (c.wk < 4 || c.wk > 16 || c.wk % 4 || c.ks < 1 || c.ks > a.K / 512) return hipErrorInvalidValue;
  const dim3 grid((unsigned)codebook_row_blocks(c, a.N), c.ks, a.M);
  const dim3 block(64 * c.wk);
  const size_t lds = PSUM_BYTES + CB_BYTES + 16;
  const bool sal = reinterpret_cast<uintptr_t>(a.scales) % 8 == 0;
  auto kern = sal ? &gemv_codebook_kernel<true> : &gemv_codebook_kernel<false>;
  static bool raised[2] = {false, false};
  if (!raised[sal]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    raised[sal] = true;
  }
  hipLaunchKernelGGL(kern, grid, block, lds, s, a);
  return hipGetLastError();
}

}  // namespace qg
