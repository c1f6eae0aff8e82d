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
//  * Codes are an [N, K/4] uint8 matrix in the tiled 8-bit device layout
//    (qgemv_pack(8, QGEMV_LAYOUT_DEVICE, N, K/4)): a 16-row x 128-code tile is
//    one contiguous 2 KB block, lane l holding row l % 16 and the 32 codes of
//    quarter l / 16, which is one quant group.  A tile therefore spans a
//    "quad" of 4 groups (128 segments, 512 k), the unit the Psumbook is built
//    for.
//  * Psumbook of a quad in LDS: fp16 P[c][s], c = centroid, s = segment in
//    the quad, 256-byte row stride (64 KB).  The address of a lookup is
//    (code << 8) | (64 kq) -- one v_perm_b32 of the code word -- plus a
//    constant offset for the segment; two lookups are summed into the fp32
//    partial by one v_dot2 against (1, 1).
//  * Work split: a workgroup holds WK waves x TPW row-tiles (16 * TPW * WK
//    weight rows) so one build serves many rows, and a K range of whole quads;
//    the K ranges of a row block are reduced in a fixed order by the last of
//    their workgroups to finish (a counter per row block in the caller's
//    workspace), so the result is deterministic.  Batch rows are grid z.
//  * Per quad: build (each thread a pair of segments for a set of centroids,
//    codebook entries broadcast from LDS) / barrier / lookups for the wave's
//    tiles, whose codes and scales were prefetched one quad ahead.
#include "common.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

constexpr uint32_t PSUM_BYTES = 256u * 256u;  // 256 centroids x 128 segments x fp16
constexpr uint32_t CB_BYTES = 256u * 4u * 2u;   // the codebook, staged

__device__ __forceinline__ float quarter_sum_cb(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t su = __float_as_uint(s);
  const auto b = __builtin_amdgcn_permlane16_swap(su, su, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int TPW>
__global__ void __launch_bounds__(1024) gemv_codebook_kernel(CodebookArgs a) {
  // LDS: [Psumbook 64 KB][codebook 2 KB][flag]
  extern __shared__ __attribute__((aligned(16))) uint32_t lsm[];
  char* const lds = reinterpret_cast<char*>(lsm);
  uint32_t* const flag = reinterpret_cast<uint32_t*>(lds + PSUM_BYTES + CB_BYTES);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int WK = blockDim.x >> 6;
  const int n = lane & 15;
  const int kq = lane >> 4;
  const int M = a.M, N = a.N, K = a.K;
  const int KC = K / 4;       // codes per row
  const int G = K / 128;      // quant groups
  const int QN = K / 512;     // quads = 128-code tiles per tile-row
  const int NT = (N + 15) / 16;
  const int m = blockIdx.z;
  const int ks = blockIdx.y, KS = gridDim.y;
  const int q0 = (QN * ks) / KS, q1 = (QN * (ks + 1)) / KS;
  const int rtw = (blockIdx.x * WK + wave) * TPW;  // first row-tile of this wave
  // (code byte << 8) | 64 kq, by byte: v_perm selectors
  const uint32_t kqw = 64u * kq;

  const rsrc_t rc = make_rsrc(a.codes, (uint32_t)NT * 16u * KC);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * G * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);

  struct St {
    u4 c[TPW][2];  // 32 codes per lane and tile (8 words)
    uint16_t s[TPW];
  };
  auto load_stage = [&](int q, St& st) {
    const bool qv = q < q1;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int rt = rtw + t;
      const bool ok = qv && rt < NT;
      const uint32_t sw = __builtin_amdgcn_readfirstlane(ok ? ((uint32_t)rt * QN + q) * 2048u : 0u);
#pragma unroll
      for (int h = 0; h < 2; ++h) st.c[t][h] = bload16<CPOL_NT>(rc, ok ? 16u * lane + 1024u * h : OOB, sw);
      const uint32_t row = (uint32_t)rt * 16u + n;
      st.s[t] = bload2(rs, ok && row < (uint32_t)N ? (row * (uint32_t)G + 4u * q + kq) * 2u : OOB);
    }
  };

  St ring[2];
  load_stage(q0, ring[0]);

  // codebook into LDS once
  for (int i = threadIdx.x; i < 512; i += blockDim.x)
    lsm[(PSUM_BYTES / 4) + i] = bload4(make_rsrc(a.codebook, CB_BYTES), 4u * i);

  float acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = 0.f;

  // build: thread -> segment pair sp (2 sp, 2 sp + 1) and centroids c = c0 + cstep * i
  const int sp = threadIdx.x & 63;
  const int c0 = threadIdx.x >> 6, cstep = WK;
  const uint32_t xrow = (uint32_t)m * K;
  const uint2* cb = reinterpret_cast<const uint2*>(lds + PSUM_BYTES);

  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  auto step = [&](int q, const St& st, St& nxt) {
    load_stage(q + 1, nxt);  // next quad (zeros past the range)
    // x of segments 2 sp, 2 sp + 1 of this quad: 8 halves
    const u4 xv = bload16(rx, (xrow + 512u * q + 8u * sp) * 2u);
    __syncthreads();  // the previous quad's lookups are done with P
    const h2 xa = as_h2(xv[0]), xb = as_h2(xv[1]), xc = as_h2(xv[2]), xd = as_h2(xv[3]);
    for (int c = c0; c < 256; c += cstep) {
      const uint2 cc = cb[c];  // C[c][0..3], broadcast
      const float p0 = dot2(as_h2(cc.y), xb, dot2(as_h2(cc.x), xa, 0.f));
      const float p1 = dot2(as_h2(cc.y), xd, dot2(as_h2(cc.x), xc, 0.f));
      lsm[c * 64 + sp] = (uint32_t)f2h(p0) | ((uint32_t)f2h(p1) << 16);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint32_t w = st.c[t][d / 4][d % 4];
        // word d holds code offsets 4d + (0, 2, 1, 3) in its bytes 0..3
        const uint32_t a0 = __builtin_amdgcn_perm(w, kqw, 0x0C0C0400u);
        const uint32_t a1 = __builtin_amdgcn_perm(w, kqw, 0x0C0C0500u);
        const uint32_t a2 = __builtin_amdgcn_perm(w, kqw, 0x0C0C0600u);
        const uint32_t a3 = __builtin_amdgcn_perm(w, kqw, 0x0C0C0700u);
        const uint32_t so = 8u * d;  // segment 4d at 2 bytes per entry
        h2 pa, pb;
        pa[0] = *reinterpret_cast<const _Float16*>(lds + a0 + so);       // segment 4d
        pa[1] = *reinterpret_cast<const _Float16*>(lds + a2 + so + 2u);  // segment 4d + 1
        pb[0] = *reinterpret_cast<const _Float16*>(lds + a1 + so + 4u);  // segment 4d + 2
        pb[1] = *reinterpret_cast<const _Float16*>(lds + a3 + so + 6u);  // segment 4d + 3
        part = dot2(pa, ones, part);
        part = dot2(pb, ones, part);
      }
      acc[t] = fmaf(h2f(st.s[t]), part, acc[t]);
    }
  };
  // two quads per iteration so the stage buffers are named statically
  for (int q = q0; q < q1; q += 2) {
    step(q, ring[0], ring[1]);
    if (q + 1 < q1) step(q + 1, ring[1], ring[0]);
  }

  // the four k-quarters of a row (groups 4q + kq) into one sum per row
  float rs_[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) rs_[t] = quarter_sum_cb(acc[t]);

  if (KS == 1) {
    if (lane < 16) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const int row = (rtw + t) * 16 + lane;
        if (row < N) a.y[(size_t)m * N + row] = f2h(rs_[t]);
      }
    }
    return;
  }
  // K split: partial sums to the workspace; the last workgroup of the row
  // block adds them in K order
  if (lane < 16) {
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int row = (rtw + t) * 16 + lane;
      if (row < N) a.ws[((size_t)ks * M + m) * N + row] = rs_[t];
    }
  }
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
    const int r0 = blockIdx.x * WK * TPW * 16;
    for (int i = threadIdx.x; i < WK * TPW * 16; i += blockDim.x) {
      const int row = r0 + i;
      if (row >= N) continue;
      float sum = 0.f;
      for (int k = 0; k < KS; ++k)
        sum += __builtin_nontemporal_load(&a.ws[((size_t)k * M + m) * N + row]);
      a.y[(size_t)m * N + row] = f2h(sum);
    }
  }
}

template <int TPW>
hipError_t launch_c(const CodebookArgs& a, const CodebookCfg& c, hipStream_t s) {
  const int NT = (a.N + 15) / 16;
  const int rb = (NT + TPW * c.wk - 1) / (TPW * c.wk);
  const dim3 grid(rb, c.ks, a.M);
  const dim3 block(64 * c.wk);
  const size_t lds = PSUM_BYTES + CB_BYTES + 16;
  static bool raised = false;
  if (!raised) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemv_codebook_kernel<TPW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    raised = true;
  }
  hipLaunchKernelGGL((gemv_codebook_kernel<TPW>), grid, block, lds, s, a);
  return hipGetLastError();
}

}  // namespace

// Workspace: KS x M x N fp32 partial sums, then one counter per (batch row,
// row block).  Counters must be zero before first use; every call leaves
// them zero.
size_t codebook_ws_bytes(const CodebookCfg& c, int M, int N) {
  if (c.ks <= 1) return 0;
  const int NT = (N + 15) / 16;
  const size_t rb = (NT + c.tpw * c.wk - 1) / (c.tpw * c.wk);
  return (size_t)c.ks * M * N * 4 + (size_t)M * rb * 4;
}

CodebookCfg pick_codebook(int M, int N, int K) {
  (void)M;
  CodebookCfg c;
  c.wk = 16;
  c.tpw = 2;
  const int NT = (N + 15) / 16;
  const int rb = (NT + c.tpw * c.wk - 1) / (c.tpw * c.wk);
  const int QN = K / 512;
  // split K until about two workgroups per CU (whole quads per split)
  c.ks = 1;
  while (c.ks < QN && (long)rb * c.ks * 2 <= 512) c.ks *= 2;
  if (c.ks > QN) c.ks = QN;
  return c;
}

hipError_t launch_gemv_codebook(const CodebookArgs& a, const CodebookCfg& c, hipStream_t s) {
  if (c.wk < 1 || c.wk > 16 || c.ks < 1) return hipErrorInvalidValue;
  switch (c.tpw) {
    case 1: return launch_c<1>(a, c, s);
    case 2: return launch_c<2>(a, c, s);
    case 4: return launch_c<4>(a, c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
