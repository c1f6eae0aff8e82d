// VALU GEMV for group-wise asymmetric WbA16 weights (b = 2, 4, 8) at small
// decode batch, on gfx950.
//
// Computes y[m, n] = sum_k x[m, k] * s[n, k/128] * (q[n, k] - z[n, k/128]) from
// the device-packed codes (32/b codes per uint32 along K; the two 16-bit halves
// of a word hold the even and the odd k of its range).  This is the weight-only group-wise asymmetric format of the QFactory
// (ATC'25) review ("Problem and motivation": fine-grained asymmetric scale/zero
// parameters; "Experiments": asymmetric W8/W4/W2, group 128x1).
//
// Design (CDNA4, memory-bound decode):
//  * Work split.  A workgroup owns RB weight rows and all of K.  Its WK waves
//    split K into chunks; inside a chunk each lane owns one 16-byte slice of a
//    row (32/b*4 consecutive k), and RI rows are covered per wave-wide load
//    (64/RI lanes per row).  Each lane keeps the activations of its slice in
//    VGPRs and reuses them for every row of the workgroup.
//  * Weights stream with one non-temporal dwordx4 per lane per row: every
//    code is read from HBM exactly once, fully coalesced.
//  * Unpack: each code field is OR-ed into the mantissa of fp16 1024.0
//    (bits 0x6400); for a field at bit offset 2c the result is exactly
//    1024 + 4^c q.  One packed fp16 FMA per pair then gives q - z exactly:
//    (1024 + 4^c q) * 4^-c - (1024 * 4^-c + z).  In the device layout the two
//    halves of such a pair are consecutive k, so they meet the activations
//    as loaded, with no shuffles.  All values are small integers,
//    so nothing is rounded before the product with x.  (The zero point is
//    subtracted before the product rather than through the group identity
//    s(sum q x - z sum x): in fp32 the identity form leaves a residue of order
//    1024 * sum|x| * 2^-24 that does not vanish when q == z.)
//  * Multiply-accumulate: v_dot2_f32_f16 into fp32, one partial per lane per
//    row; the lane's slice lies inside one 128-group, so the group scale is
//    applied once per lane and row (QFactory review, observation 1: scale and
//    zero shared by the group are loaded once, not per element).
//  * K reduction: DPP adds across the lanes of a row, then across the waves of
//    the workgroup through LDS, in a fixed order (bitwise deterministic).
#include "common.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

// ---------------------------------------------------------------------------
// unpack + exact zero-point subtraction, per 32-bit word of codes.
// deq() writes PPD fp16 pairs: pair i holds fields (i, i + PPD), which in the
// device layout are k offsets (2i, 2i + 1) of the word.  `mg` is a VGPR holding
// fp16x2 (1024, 1024).
// ---------------------------------------------------------------------------
template <int BITS>
struct Uni;

template <>
struct Uni<4> {
  static constexpr int CPD = 8;  // codes per word
  struct Z {
    h2 c1, c16;
  };
  static __device__ __forceinline__ Z zc(uint32_t z) {
    const uint32_t zp = z | (z << 16);
    return {as_h2(zp | 0x64006400u),           // 1024 + z
            as_h2((zp << 4) | 0x54005400u)};   // 64 + z
  }
  static __device__ __forceinline__ void deq(uint32_t w, uint32_t mg, const Z& z, h2* d) {
    const h2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const uint32_t u = w >> 8;
    d[0] = as_h2(and_or(w, 0x000F000Fu, mg)) - z.c1;              // fields 0, 4
    d[1] = fma2(as_h2(and_or(w, 0x00F000F0u, mg)), k16, -z.c16);  // fields 1, 5
    d[2] = as_h2(and_or(u, 0x000F000Fu, mg)) - z.c1;              // fields 2, 6
    d[3] = fma2(as_h2(and_or(u, 0x00F000F0u, mg)), k16, -z.c16);  // fields 3, 7
  }
};

template <>
struct Uni<8> {
  static constexpr int CPD = 4;
  struct Z {
    h2 c1;
  };
  static __device__ __forceinline__ Z zc(uint32_t z) {
    const uint32_t zp = z | (z << 16);
    return {as_h2(zp | 0x64006400u)};  // 1024 + z
  }
  static __device__ __forceinline__ void deq(uint32_t w, uint32_t, const Z& z, h2* d) {
    // byte permute: (b0, 0x64, b2, 0x64) and (b1, 0x64, b3, 0x64) -> 1024 + q
    d[0] = as_h2(__builtin_amdgcn_perm(0x64646464u, w, 0x04020400u)) - z.c1;  // bytes 0, 2
    d[1] = as_h2(__builtin_amdgcn_perm(0x64646464u, w, 0x04030401u)) - z.c1;  // bytes 1, 3
  }
};

template <>
struct Uni<2> {
  static constexpr int CPD = 16;
  struct Z {
    h2 c[5];
  };
  static __device__ __forceinline__ Z zc(uint32_t z) {
    const uint32_t zp = z | (z << 16);
    Z r;
    r.c[0] = as_h2(zp | 0x64006400u);         // 1024 + z
    r.c[1] = as_h2((zp << 2) | 0x5C005C00u);  //  256 + z
    r.c[2] = as_h2((zp << 4) | 0x54005400u);  //   64 + z
    r.c[3] = as_h2((zp << 6) | 0x4C004C00u);  //   16 + z
    r.c[4] = as_h2((zp << 8) | 0x44004400u);  //    4 + z
    return r;
  }
  static __device__ __forceinline__ void deq(uint32_t w, uint32_t mg, const Z& z, h2* d) {
    const h2 q1 = {(_Float16)0.25f, (_Float16)0.25f};
    const h2 q2 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 q3 = {(_Float16)0.015625f, (_Float16)0.015625f};
    const h2 q4 = {(_Float16)0.00390625f, (_Float16)0.00390625f};
    const uint32_t u = w >> 10;
    d[0] = as_h2(and_or(w, 0x00030003u, mg)) - z.c[0];
    d[1] = fma2(as_h2(and_or(w, 0x000C000Cu, mg)), q1, -z.c[1]);
    d[2] = fma2(as_h2(and_or(w, 0x00300030u, mg)), q2, -z.c[2]);
    d[3] = fma2(as_h2(and_or(w, 0x00C000C0u, mg)), q3, -z.c[3]);
    d[4] = fma2(as_h2(and_or(w, 0x03000300u, mg)), q4, -z.c[4]);
    d[5] = as_h2(and_or(u, 0x00030003u, mg)) - z.c[0];
    d[6] = fma2(as_h2(and_or(u, 0x000C000Cu, mg)), q1, -z.c[1]);
    d[7] = fma2(as_h2(and_or(u, 0x00300030u, mg)), q2, -z.c[2]);
  }
};


// One pipeline stage of weight rows for one lane: NV 16-byte code vectors,
// the zero-point word and the scale of each of U row groups.
template <int U, int NV>
struct Stage {
  u4 w[U][NV];
  uint32_t z[U];
  uint16_t s[U];
};

template <int BITS, int MT, int RI, int NV, int U>
__global__ void __launch_bounds__(NV == 1 ? 1024 : 512) gemv_valu_kernel(UniformArgs a, int RB) {
  using T = Uni<BITS>;
  constexpr int SL = NV * 128 / BITS;  // k per lane slice (NV x 16 bytes of codes)
  constexpr int LPR = 64 / RI;         // lanes per weight row
  constexpr int CK = LPR * SL;         // k per chunk
  constexpr int PPD = T::CPD / 2;      // fp16 pairs per code word
  constexpr int NW = 4 * NV;           // code words per lane slice
  constexpr int NP = NW * PPD;         // pairs per lane slice
  constexpr int ZPW = 32 / BITS;       // zero points per uint32
  constexpr uint32_t ZMASK = (1u << BITS) - 1u;
  static_assert(SL <= 128, "a lane slice must stay inside one quant group");

  extern __shared__ float red[];  // [WK][RB][MT]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int WK = blockDim.x >> 6;
  const int sub = lane / LPR;
  const int kl = lane % LPR;
  const int n0 = blockIdx.x * RB;
  const int m0 = blockIdx.y * MT;
  const int M = a.M, N = a.N, K = a.K;
  const int NC = (K + CK - 1) / CK;
  const int G = K / 128;
  const uint32_t wrow = (uint32_t)K * BITS / 8;      // code bytes per row
  const uint32_t zrow = 4u * ((G * BITS + 31) / 32); // zero-point bytes per row
  const int nrg = RB / RI;                           // row groups per workgroup
  const uint32_t mg = magic1024x2();

  // bounds-checked views: rows >= N read as zero (scale 0 => no contribution)
  const rsrc_t rw = make_rsrc(a.wq, (uint32_t)N * wrow);
  const rsrc_t rz = make_rsrc(a.zeros, (uint32_t)N * zrow);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * G * 2u);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)M * K * 2u);

  float* myred = red + (size_t)wave * RB * MT;
  if (wave >= NC) {
    for (int i = lane; i < RB * MT; i += 64) myred[i] = 0.f;
  }

  for (int c = wave; c < NC; c += WK) {
    const bool first = (c == wave);
    const int k0 = c * CK + kl * SL;
    const bool kact = k0 < K;  // lanes past K see x = 0 and scale 0
    const int g = kact ? k0 / 128 : 0;
    const int zshift = BITS * (g % ZPW);

    // byte offsets of row (n0 + sub); one row group = RI rows
    const uint32_t row0 = (uint32_t)(n0 + sub);
    const uint32_t woff0 = kact ? row0 * wrow + (uint32_t)k0 * BITS / 8 : OOB;
    const uint32_t zoff0 = row0 * zrow + 4u * (uint32_t)(g / ZPW);
    const uint32_t soff0 = kact ? (row0 * (uint32_t)G + (uint32_t)g) * 2u : OOB;
    const uint32_t wstep = RI * wrow, zstep = RI * zrow, sstep = RI * (uint32_t)G * 2u;

    auto load_stage = [&](int rg0, Stage<U, NV>& st) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t rg = (uint32_t)(rg0 + u);
#pragma unroll
        for (int v = 0; v < NV; ++v) st.w[u][v] = bload16<CPOL_NT>(rw, woff0 + 16u * v, rg * wstep);
        st.z[u] = bload4(rz, zoff0, rg * zstep);
        st.s[u] = bload2(rs, soff0, rg * sstep);
      }
    };

    // weights first: the first stage is in flight while the activations load
    Stage<U, NV> sa, sb;
    load_stage(0, sa);

    // activations of this slice: pair p = (x[k0 + 2p], x[k0 + 2p + 1]) is the
    // operand of unpacked pair p, as loaded
    h2 X[MT][NP];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint32_t xoff = (kact && m0 + m < M) ? ((uint32_t)(m0 + m) * K + k0) * 2u : OOB;
#pragma unroll
      for (int v = 0; v < SL / 8; ++v) {
        const u4 t = bload16(rx, xoff + 16u * v);
#pragma unroll
        for (int e = 0; e < 4; ++e) X[m][4 * v + e] = as_h2(t[e]);
      }
    }

    auto compute_stage = [&](int rg0, const Stage<U, NV>& st) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const typename T::Z zz = T::zc((st.z[u] >> zshift) & ZMASK);
        float part[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) part[m] = 0.f;
#pragma unroll
        for (int d = 0; d < NW; ++d) {
          h2 q[PPD];
          T::deq(st.w[u][d / 4][d % 4], mg, zz, q);
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < PPD; ++i) part[m] = dot2(q[i], X[m][d * PPD + i], part[m]);
        }
        const float s = h2f(st.s[u]);
        const int r = (rg0 + u) * RI + sub;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const float v = group_sum<LPR>(s * part[m]);
          if (kl == LPR - 1) {
            if (first)
              myred[r * MT + m] = v;
            else
              myred[r * MT + m] += v;
          }
        }
      }
    };

    // two stages in flight: load stage i+1 while computing stage i
    for (int rg0 = 0; rg0 < nrg; rg0 += 2 * U) {
      if (rg0 + U < nrg) load_stage(rg0 + U, sb);
      compute_stage(rg0, sa);
      if (rg0 + U >= nrg) break;
      if (rg0 + 2 * U < nrg) load_stage(rg0 + 2 * U, sa);
      compute_stage(rg0 + U, sb);
    }
  }

  __syncthreads();
  for (int i = threadIdx.x; i < RB * MT; i += blockDim.x) {
    const int m = i / RB, r = i % RB;
    float sum = 0.f;
    for (int w = 0; w < WK; ++w) sum += red[((size_t)w * RB + r) * MT + m];
    if (n0 + r < N && m0 + m < M) a.y[(size_t)(m0 + m) * N + n0 + r] = f2h(sum);
  }
}

template <int BITS, int MT, int RI, int NV, int U>
hipError_t launch_t(const UniformArgs& a, const ValuCfg& c, hipStream_t s) {
  const dim3 grid((a.N + c.rb - 1) / c.rb, (a.M + MT - 1) / MT);
  const dim3 block(64 * c.wk);
  const size_t lds = (size_t)c.wk * c.rb * MT * sizeof(float);
  hipLaunchKernelGGL((gemv_valu_kernel<BITS, MT, RI, NV, U>), grid, block, lds, s, a, c.rb);
  return hipGetLastError();
}

template <int BITS, int MT, int RI, int NV>
hipError_t launch_u(const UniformArgs& a, const ValuCfg& c, hipStream_t s) {
  switch (c.u) {
    case 2: return launch_t<BITS, MT, RI, NV, 2>(a, c, s);
    case 4: return launch_t<BITS, MT, RI, NV, 4>(a, c, s);
  }
  return hipErrorInvalidValue;
}

template <int BITS, int MT, int RI>
hipError_t launch_nv(const UniformArgs& a, const ValuCfg& c, hipStream_t s) {
  switch (c.nv) {
    case 1: return launch_u<BITS, MT, RI, 1>(a, c, s);
    case 2: return launch_u<BITS, MT, RI, 2>(a, c, s);
  }
  return hipErrorInvalidValue;
}

template <int BITS, int MT>
hipError_t launch_ri(const UniformArgs& a, const ValuCfg& c, hipStream_t s) {
  switch (c.ri) {
    case 1: return launch_nv<BITS, MT, 1>(a, c, s);
    case 2: return launch_nv<BITS, MT, 2>(a, c, s);
    case 4: return launch_nv<BITS, MT, 4>(a, c, s);
  }
  return hipErrorInvalidValue;
}

template <int BITS>
hipError_t launch_mt(const UniformArgs& a, const ValuCfg& c, hipStream_t s) {
  switch (c.mt) {
    case 1: return launch_ri<BITS, 1>(a, c, s);
    case 2: return launch_ri<BITS, 2>(a, c, s);
    case 4: return launch_ri<BITS, 4>(a, c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Launch shape from measured sweeps on MI355X (graph-timed, cache-cold
// weights): K is split into 8..16 chunks of 64/RI lanes x 16 bytes, one wave
// per chunk (16 at most, looping beyond); workgroups cover the fewest rows that
// keep the grid at or below ~2048 workgroups, two row groups per stage.
ValuCfg pick_valu(int bits, int M, int N, int K) {
  ValuCfg c;
  c.mt = M <= 1 ? 1 : (M <= 2 ? 2 : 4);
  c.nv = 1;
  c.u = 2;
  const int SL = 128 / bits;  // k per 16-byte lane slice
  auto chunks = [&](int ri) { return (K + (64 / ri) * SL - 1) / ((64 / ri) * SL); };
  c.ri = 4;
  if (chunks(4) > 8 && chunks(2) <= 8) c.ri = 2;
  if (chunks(4) > 16 && chunks(2) > 16 && chunks(2) <= 32) c.ri = 2;
  if (chunks(2) > 32) c.ri = 1;
  const int nc = chunks(c.ri);
  c.wk = nc < 16 ? nc : 16;
  const int step = c.ri * c.u;
  const int mtiles = (M + c.mt - 1) / c.mt;
  int rb = step;
  while (rb < 256 && (long)((N + rb - 1) / rb) * mtiles > 2048) rb += step;
  c.rb = rb;
  return c;
}

hipError_t launch_gemv_valu(const UniformArgs& a, const ValuCfg& c, hipStream_t s) {
  if (c.u != 2 && c.u != 4) return hipErrorInvalidValue;
  if (c.wk < 1 || c.wk > 16 || c.rb < 1 || c.rb % (c.ri * c.u)) return hipErrorInvalidValue;
  if (c.nv * 128 / a.bits > 128 || c.wk * 64 > (c.nv == 1 ? 1024 : 512)) return hipErrorInvalidValue;
  if (c.ri != 1 && c.ri != 2 && c.ri != 4) return hipErrorInvalidValue;
  switch (a.bits) {
    case 2: return launch_mt<2>(a, c, s);
    case 4: return launch_mt<4>(a, c, s);
    case 8: return launch_mt<8>(a, c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
