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
// shared by the workgroup.
//
// Block: 32 MI activation rows x 64 weight rows (4 tile-rows), 4 waves; wave
// w owns tile-row w of the block and every activation row of it, so each
// weight fragment is dequantized once per workgroup (the four waves each read
// the A fragments from LDS).  Per group a wave runs 8 MI MFMAs into group
// partials and adds each times the lane's row scale (one rounding per group,
// as the decode kernels).  Deterministic.
#include "common.hpp"
#include "dequant.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

constexpr int XROW = 136;  // staged activation row: 128 halves + 8 of padding (bank spread)

template <int BITS, int MI>
__global__ void __launch_bounds__(256) gemm_tiles_kernel(UniformArgs a) {
  constexpr int NMI = 2 * MI;  // 16-row activation tiles per wave (all of the block)
  using TR = Uni<BITS>;
  constexpr int PPD = TR::CPD / 2;
  constexpr int ZPW = 32 / BITS;
  constexpr uint32_t TB = 16u * 128u * BITS / 8;  // tile bytes
  constexpr int BM = 32 * MI;                     // activation rows per block
  constexpr int XP = BM * 16 / 256;               // 16-byte staging pieces per thread
  __shared__ __attribute__((aligned(16))) _Float16 xs[2][BM * XROW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kq = lane >> 4;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / 128;
  const int NT = (N + 15) / 16;
  const uint32_t zrow = 4u * ((G * BITS + 31) / 32);
  const int m0 = blockIdx.y * BM;
  const int rt = blockIdx.x * 4 + wave;  // this wave's tile-row
  const uint32_t mg = magic1024x2();

  const rsrc_t rw = make_rsrc(a.wq, (uint32_t)NT * G * TB);
  const rsrc_t rz = make_rsrc(a.zeros, (uint32_t)N * zrow);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * G * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);

  // activation staging: thread t moves 16-byte pieces t, t + 256, ... of the
  // block's BM x 128 tile of group g (rows past M read zeros)
  auto x_load = [&](int g, u4 (&v)[XP]) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int idx = threadIdx.x + 256 * i, r = idx >> 4, c8 = idx & 15;
      v[i] = bload16(rx, m0 + r < M ? ((uint32_t)(m0 + r) * K + 128u * g + 8u * c8) * 2u : OOB);
    }
  };
  auto x_store = [&](int b, const u4 (&v)[XP]) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int idx = threadIdx.x + 256 * i, r = idx >> 4, c8 = idx & 15;
      *reinterpret_cast<u4*>(&xs[b][r * XROW + 8 * c8]) = v[i];
    }
  };
  // weights of the wave's tile-row in group g: codes, scale and zero point
  struct Wst {
    uint32_t w[BITS];
    uint16_t s;
    uint32_t z;
  };
  const bool tv = rt < NT;
  const int row = 16 * rt + n;
  const bool rv = tv && row < N;
  auto w_load = [&](int g, Wst& st) {
    const uint32_t tb = ((uint32_t)rt * G + g) * TB;
    if constexpr (BITS == 2) {
      const u2 v = __builtin_bit_cast(
          u2, __builtin_amdgcn_raw_buffer_load_b64(rw, tv ? tb + 8u * lane : OOB, 0, CPOL_NT));
      st.w[0] = v.x;
      st.w[1] = v.y;
    } else {
#pragma unroll
      for (int h = 0; h < BITS / 4; ++h) {
        const u4 v = bload16<CPOL_NT>(rw, tv ? tb + 1024u * h + 16u * lane : OOB);
#pragma unroll
        for (int e = 0; e < 4; ++e) st.w[4 * h + e] = v[e];
      }
    }
    st.s = bload2(rs, rv ? ((uint32_t)row * G + g) * 2u : OOB);
    st.z = bload4(rz, rv ? (uint32_t)row * zrow + 4u * (uint32_t)(g / ZPW) : OOB);
  };

  f4 acc[NMI];
#pragma unroll
  for (int i = 0; i < NMI; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};

  // Pipeline, distance 2: group g is computed from LDS buffer g % 2 while
  // group g + 1 waits in registers (stored to the other buffer after the
  // compute) and group g + 2 is being loaded; the barrier waits for LDS
  // traffic only, so those loads stay in flight across it.
  u4 xv[2][XP];
  Wst wst[3];
  x_load(0, xv[0]);
  w_load(0, wst[0]);
  x_load(1, xv[1]);  // (with one group: other data in bounds, never used)
  w_load(1, wst[1]);
  x_store(0, xv[0]);
  __syncthreads();

  auto step = [&](int g, int b, u4 (&xnext)[XP], u4 (&xlater)[XP], const Wst& cur, Wst& later) {
    if (g + 2 < G) {  // (workgroup-uniform)
      x_load(g + 2, xlater);
      w_load(g + 2, later);
    }
    // B fragments: the (q - z) pairs of the lane's 32 k
    h2 p[16];
    const typename TR::Z zz = TR::zc((cur.z >> (BITS * (g % ZPW))) & ((1u << BITS) - 1u));
#pragma unroll
    for (int d = 0; d < BITS; ++d) TR::deq(cur.w[d], mg, zz, p + d * PPD);
    const float sc = h2f(cur.s);  // lane l: weight row l % 16
#pragma unroll
    for (int i = 0; i < NMI; ++i) {
      // A fragments: block row 16 i + n, k 32 kq + 8 s .. + 7 of the group
      const _Float16* xr = &xs[b][(16 * i + n) * XROW + 32 * kq];
      f4 dd = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const h8 av = __builtin_bit_cast(h8, *reinterpret_cast<const u4*>(xr + 8 * s));
        const u4 bv = {as_u32(p[4 * s]), as_u32(p[4 * s + 1]), as_u32(p[4 * s + 2]), as_u32(p[4 * s + 3])};
        dd = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(h8, bv), dd, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][r] = fmaf(sc, dd[r], acc[i][r]);
    }
    if (g + 1 < G) x_store(b ^ 1, xnext);
    lds_barrier();  // group g + 1 staged; every wave is done with buffer b
  };
  // six groups per iteration so the register stages are named statically
  for (int g = 0; g < G; g += 6) {
    step(g, 0, xv[1], xv[0], wst[0], wst[2]);
    if (g + 1 < G) step(g + 1, 1, xv[0], xv[1], wst[1], wst[0]);
    if (g + 2 < G) step(g + 2, 0, xv[1], xv[0], wst[2], wst[1]);
    if (g + 3 < G) step(g + 3, 1, xv[0], xv[1], wst[0], wst[2]);
    if (g + 4 < G) step(g + 4, 0, xv[1], xv[0], wst[1], wst[0]);
    if (g + 5 < G) step(g + 5, 1, xv[0], xv[1], wst[2], wst[1]);
  }

  // lane l holds D[row 4 (l / 16) + r][weight row l % 16] of each 16 x 16 tile
#pragma unroll
  for (int i = 0; i < NMI; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + 16 * i + 4 * kq + r;
      if (m < M && row < N) a.y[(size_t)m * N + row] = f2h(acc[i][r]);
    }
}

}  // namespace

template <int MI>
hipError_t launch_mi(const UniformArgs& a, hipStream_t s) {
  const int NT = (a.N + 15) / 16;
  const dim3 grid((NT + 3) / 4, (a.M + 32 * MI - 1) / (32 * MI)), block(256);
  switch (a.bits) {
    case 2: hipLaunchKernelGGL((gemm_tiles_kernel<2, MI>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemm_tiles_kernel<4, MI>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((gemm_tiles_kernel<8, MI>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_tiles(const UniformArgs& a, int mi, hipStream_t s) {
  if (mi == 2) return launch_mi<2>(a, s);
  if (mi == 4) return launch_mi<4>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace qg
