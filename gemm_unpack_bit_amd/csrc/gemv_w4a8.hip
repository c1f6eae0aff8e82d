// W4A8 GEMV (ADAngel review: arbitrary-precision quantization such as W4A8;
// DPR, decomposition / partial product / reconstruction, with its padding
// and split strategies), three ways on gfx950:
//
//  * padding (int8 matrix cores): symmetric int8 activations,
//      x_q[m, k] = rint(x[m, k] / s_x[m]) clamped to [-127, 127],
//      s_x[m] = max_k |x[m, k]| / 127                        (fp32)
//    the 4-bit codes padded to the signed bytes q - z:
//      y[m, n] = s_x[m] * sum_g s_w[n, g] * sum_{k in g} (q[n, k] - z[n, g]) x_q[m, k]
//  * split (fp8 matrix cores): the same activations and result, with each
//    int8 activation decomposed into a signed high and an unsigned low
//    4-bit slice, x_q = 16 h + l.  Each slice (16 h, l) and each q - z is a
//    small integer, exact in fp8 e4m3, so v_mfma_f32_16x16x128_f8f6f4 forms
//    the two partial products exactly and one accumulator adds them (the
//    factor 16 travels in the high slice's exponent): the reconstruction is
//    exact and the result is bit for bit the padding strategy's.
//  * asymmetric activations (int8 matrix cores): one scale and one zero
//    point per row (range widened to contain 0),
//      s_x = (hi - lo) / 255, zx = -128 - rint(lo / s_x), x_q = rint(x / s_x) + zx,
//    and the raw codes q as the B operand, no per-element zero point on either
//    side: per group the QFactory zero-point expansion (review, observation 2)
//      sum (q - z)(x_q - zx) = sum q x_q - z sum x_q - zx sum q + 128 z zx
//    with sum x_q from the quantization kernel and sum q from v_dot8 on the
//    packed codes, every term an exact integer.
//
// Two kernels on the caller's stream:
//  * quant_rows_kernel<MODE>: writes the activations (and slices, sums, zero
//    points) and s_x to the caller's workspace; fp32 correctly rounded
//    division and round-to-nearest-even, so every integer is the one the
//    definition gives.  Each workgroup takes 2048 k of one row: it reads the
//    whole row for the range (exact in any order, so every workgroup of the
//    row finds the same s_x) and quantizes its own part, which it already
//    holds in registers.
//  * gemv_w4a8_kernel<TR, MODE>: a workgroup owns TR (1 or 2) 16-row
//    tile-rows of the 4-bit tiled device layout; its waves take runs of WU
//    quant groups round-robin, issuing all of a run's loads before its
//    MFMAs.  A lane's 4 code words hold its row's 32 k of the group.  The
//    group sums are exact; each is scaled by the lane's row scale, the waves
//    are added in a fixed order through LDS, and the row's activation scale
//    is applied last.  Deterministic.
#include <cstdlib>
#include <mutex>

#include "common.hpp"
#include "dequant.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef short s2 __attribute__((ext_vector_type(2)));

constexpr int QT = 256;  // threads of the quantization kernel; one 8-k piece each
constexpr int QU = 4;    // pieces per thread in flight in the max pass

__device__ __forceinline__ float h8_absmax(u4 v) {
  float r = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) r = fmaxf(r, fmaxf(fabsf(h2f((uint16_t)v[e])), fabsf(h2f((uint16_t)(v[e] >> 16)))));
  return r;
}
// int8 code of one activation (s > 0): rint(x / s) clamped, as a byte
__device__ __forceinline__ uint32_t q8(uint16_t xh, float s) {
  const float v = fminf(fmaxf(rintf(h2f(xh) / s), -127.f), 127.f);  // correctly rounded fp32 division
  return (uint32_t)(int)v & 0xFFu;
}

// fp8 e4m3 bytes of two small integers (exact: |v| <= 128, at most 4
// significant bits), written into the low or high 16 bits of `old`
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair(float a, float b, uint32_t old) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(s2, old), a, b, 1.0f, HI));
}

// grid: (K / 2048 rounded up, M)
template <int MODE>
__global__ void __launch_bounds__(QT) quant_rows_kernel(W4A8Args a) {
  __shared__ float wmax[QT / 64], wmin[QT / 64];
  const int m = blockIdx.y, K = a.K, tid = threadIdx.x;
  const int np = K / 8;                       // 16-byte pieces of the row
  const int mine = blockIdx.x * QT + tid;     // the piece this thread quantizes
  const rsrc_t rx = make_rsrc(a.x + (size_t)m * K, (uint32_t)K * 2u);
  u4 own = u4{0u, 0u, 0u, 0u};
  float amax = 0.f, vmin = 0.f, vmax = 0.f;  // (the asymmetric range contains 0)
  for (int base = tid; base < np; base += QT * QU) {
    u4 v[QU];
#pragma unroll
    for (int j = 0; j < QU; ++j) {
      const int p = base + QT * j;
      v[j] = bload16(rx, p < np ? 16u * p : OOB);  // (past the row: zeros)
    }
#pragma unroll
    for (int j = 0; j < QU; ++j) {
      if constexpr (MODE == W4A8_ASYM) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = h2f((uint16_t)(v[j][e / 2] >> (16 * (e % 2))));
          vmin = fminf(vmin, f);
          vmax = fmaxf(vmax, f);
        }
      } else {
        amax = fmaxf(amax, h8_absmax(v[j]));
      }
      if (base + QT * j == mine) own = v[j];
    }
  }
  // range over the workgroup (exact, any order)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    vmin = fminf(vmin, __shfl_xor(vmin, off, 64));
    vmax = fmaxf(vmax, __shfl_xor(vmax, off, 64));
  }
  if ((tid & 63) == 0) {
    wmax[tid >> 6] = MODE == W4A8_ASYM ? vmax : amax;
    wmin[tid >> 6] = vmin;
  }
  __syncthreads();
  amax = 0.f;
  vmin = 0.f;
#pragma unroll
  for (int w = 0; w < QT / 64; ++w) {
    amax = fmaxf(amax, wmax[w]);
    vmin = fminf(vmin, wmin[w]);
  }
  if constexpr (MODE == W4A8_ASYM) {
    const float s = (amax - vmin) / 255.0f;  // correctly rounded fp32 division
    const int zx = s > 0.f ? (int)fminf(fmaxf(-128.0f - rintf(vmin / s), -128.f), 127.f) : 0;
    int sum = 0;
    if (mine < np) {
      uint32_t lo = 0u, hi = 0u;
      if (s > 0.f) {  // a zero row quantizes to zeros
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float f = h2f((uint16_t)(own[e / 2] >> (16 * (e % 2))));
          const int qv = (int)fminf(fmaxf(rintf(f / s) + (float)zx, -128.f), 127.f);
          sum += qv;
          const uint32_t b = (uint32_t)qv & 0xFFu;
          if (e < 4) lo |= b << (8 * e);
          else hi |= b << (8 * (e - 4));
        }
      }
      *reinterpret_cast<uint2*>(a.xq + (size_t)m * K + 8 * (size_t)mine) = uint2{lo, hi};
    }
    // the group's sum of x_q: 16 consecutive pieces (threads) per 128 k
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 16);
    if ((tid & 15) == 0 && mine < np) a.xsum[(mine / 16) * 16 + m] = sum;
    if (blockIdx.x == 0 && tid == 0) {
      a.sx[m] = s;
      a.zx[m] = zx;
    }
  } else {
    const float s = amax / 127.0f;  // correctly rounded fp32 division
    if (mine < np) {
      uint32_t lo = 0u, hi = 0u;
      if (s > 0.f) {  // a zero row quantizes to zeros
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          lo |= (q8((uint16_t)own[e], s) | q8((uint16_t)(own[e] >> 16), s) << 8) << (16 * e);
          hi |= (q8((uint16_t)own[2 + e], s) | q8((uint16_t)(own[2 + e] >> 16), s) << 8) << (16 * e);
        }
      }
      if constexpr (MODE == W4A8_SPLIT) {
        // x_q = 16 h + l: the slices 16 h (signed) and l (0..15) as fp8
        uint32_t hs[2] = {0u, 0u}, ls[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t wv = e < 4 ? lo : hi;
          const int b0 = (int)(int8_t)(wv >> (8 * (e % 4))), b1 = (int)(int8_t)(wv >> (8 * (e % 4 + 1)));
          const int h0 = b0 >> 4, h1 = b1 >> 4;  // arithmetic: floor(x_q / 16)
          if (e % 4 == 0) {
            hs[e / 4] = fp8_pair<false>((float)(16 * h0), (float)(16 * h1), hs[e / 4]);
            ls[e / 4] = fp8_pair<false>((float)(b0 - 16 * h0), (float)(b1 - 16 * h1), ls[e / 4]);
          } else {
            hs[e / 4] = fp8_pair<true>((float)(16 * h0), (float)(16 * h1), hs[e / 4]);
            ls[e / 4] = fp8_pair<true>((float)(b0 - 16 * h0), (float)(b1 - 16 * h1), ls[e / 4]);
          }
        }
        *reinterpret_cast<uint2*>(a.xq + (size_t)m * K + 8 * (size_t)mine) = uint2{hs[0], hs[1]};
        *reinterpret_cast<uint2*>(a.xl + (size_t)m * K + 8 * (size_t)mine) = uint2{ls[0], ls[1]};
      } else {
        *reinterpret_cast<uint2*>(a.xq + (size_t)m * K + 8 * (size_t)mine) = uint2{lo, hi};
      }
    }
    if (blockIdx.x == 0 && tid == 0) a.sx[m] = s;
  }
}

// the 8 codes of a device-layout word in k order, minus the zero point, as
// signed bytes: fields 0..7 sit at k offsets 0, 2, 4, 6, 1, 3, 5, 7
__device__ __forceinline__ uint2 codes_minus_z(uint32_t w, uint32_t z4) {
  const uint32_t lo = w & 0x0F0F0F0Fu;         // bytes: k 0, 4, 1, 5
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // bytes: k 2, 6, 3, 7
  const uint32_t k03 = __builtin_amdgcn_perm(hi, lo, 0x06040200u);  // k 0, 1, 2, 3
  const uint32_t k47 = __builtin_amdgcn_perm(hi, lo, 0x07050301u);  // k 4, 5, 6, 7
  // per byte: (q + 128 - z) stays in [113, 143] (no borrow), then ^ 0x80 = q - z
  return uint2{((k03 | 0x80808080u) - z4) ^ 0x80808080u, ((k47 | 0x80808080u) - z4) ^ 0x80808080u};
}

// the 8 codes of a device-layout word in k order as unsigned bytes (0..15)
__device__ __forceinline__ uint2 codes_raw(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  return uint2{__builtin_amdgcn_perm(hi, lo, 0x06040200u), __builtin_amdgcn_perm(hi, lo, 0x07050301u)};
}

// the lane's 32 codes of a group (4 device-layout words) as 32 fp8 e4m3
// bytes of q - z in k order: exact fp16 (q - z) pairs (dequant.hpp), then
// converted pair by pair (|q - z| <= 15: exact in e4m3)
__device__ __forceinline__ v8i codes_minus_z_fp8(const u4& w, uint32_t z, uint32_t mg) {
  const Uni<4>::Z zz = Uni<4>::zc(z);
  h2 p[16];
#pragma unroll
  for (int d = 0; d < 4; ++d) Uni<4>::deq(w[d], mg, zz, p + 4 * d);
  v8i b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s2 r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, p[2 * j], 1.0f, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r, p[2 * j + 1], 1.0f, true);
    b[j] = __builtin_bit_cast(int, r);
  }
  return b;
}

// integer sum of the values of lanes n, n + 16, n + 32, n + 48 (all four get it)
__device__ __forceinline__ uint32_t quarter_sum_u(uint32_t u) {
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t s = a[0] + a[1];
  const auto b = __builtin_amdgcn_permlane16_swap(s, s, false, false);
  return b[0] + b[1];
}

constexpr int WU = 4;  // quant groups per wave whose loads are in flight together

// TR tile-rows per workgroup (1, 2): with 2, each A fragment loaded from L2
// serves both tile-rows, halving the activation reads (they reach twice the
// weight bytes at M = 16).
template <int TR, int MODE>
__global__ void __launch_bounds__(1024) gemv_w4a8_kernel(W4A8Args a) {
  extern __shared__ __attribute__((aligned(16))) float red[];  // [WK][TR][64] float4
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int WK = blockDim.x >> 6;
  const int n = lane & 15, kq = lane >> 4;
  const int M = a.M, N = a.N, K = a.K;
  const int G = K / 128;
  const int NT = (N + 15) / 16;
  const int rt0 = blockIdx.x * TR;
  const uint32_t zrow = 4u * ((G * 4 + 31) / 32);
  const rsrc_t rw = make_rsrc(a.wq, (uint32_t)NT * G * 1024u);
  const rsrc_t rs = make_rsrc(a.scales, (uint32_t)N * G * 2u);
  const rsrc_t rz = make_rsrc(a.zeros, (uint32_t)N * zrow);
  const rsrc_t rx = make_rsrc(a.xq, (uint32_t)M * K);
  const rsrc_t rl = make_rsrc(a.xl, MODE == W4A8_SPLIT ? (uint32_t)M * K : 0u);
  const rsrc_t rq = make_rsrc(a.xsum, MODE == W4A8_ASYM ? (uint32_t)G * 64u : 0u);
  const uint32_t mg = magic1024x2();
  // A: activation row n (rows past M read zeros), the lane's 32 k of a group
  const uint32_t xo = n < M ? (uint32_t)n * K + 32u * kq : OOB;
  // asymmetric activations: the zero points of the lane's result rows 4 kq + i
  // (the 16-entry arrays hold 0 past M)
  int zxl[4] = {0, 0, 0, 0};
  if constexpr (MODE == W4A8_ASYM) {
    const u4 zv = bload16(make_rsrc(a.zx, 64u), 16u * kq);
#pragma unroll
    for (int i = 0; i < 4; ++i) zxl[i] = (int)zv[i];
  }
  // G a multiple of WU: a run's WU scales are one aligned 8-byte load and its
  // zero points one word (runs start at multiples of WU = 4, inside one
  // 8-group zero word); otherwise one load per group.
  const bool packed = G % WU == 0;

  f4 acc[TR];
#pragma unroll
  for (int t = 0; t < TR; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  for (int g0 = WU * wave; g0 < G; g0 += WU * WK) {  // (wave-uniform)
    // all loads of the run first; groups past G and tile-rows past NT read
    // zeros (scale 0: no effect)
    u4 w[TR][WU], x0[WU], x1[WU], l0[MODE == W4A8_SPLIT ? WU : 1], l1[MODE == W4A8_SPLIT ? WU : 1];
    u4 xs[MODE == W4A8_ASYM ? WU : 1];
    uint16_t sb[TR][WU];
    uint32_t zw[TR][WU];
#pragma unroll
    for (int t = 0; t < TR; ++t)
#pragma unroll
      for (int u = 0; u < WU; ++u) {
        const int g = g0 + u;
        w[t][u] = bload16<CPOL_NT>(rw, g < G && rt0 + t < NT ? ((uint32_t)(rt0 + t) * G + g) * 1024u + 16u * lane
                                                             : OOB);
      }
#pragma unroll
    for (int u = 0; u < WU; ++u) {
      const int g = g0 + u;
      x0[u] = bload16(rx, g < G ? xo : OOB, 128u * g);
      x1[u] = bload16(rx, g < G ? xo : OOB, 128u * g + 16u);
      if constexpr (MODE == W4A8_SPLIT) {
        l0[u] = bload16(rl, g < G ? xo : OOB, 128u * g);
        l1[u] = bload16(rl, g < G ? xo : OOB, 128u * g + 16u);
      }
      if constexpr (MODE == W4A8_ASYM) xs[u] = bload16(rq, g < G ? 64u * g + 16u * kq : OOB);
    }
#pragma unroll
    for (int t = 0; t < TR; ++t) {
      const int row = 16 * (rt0 + t) + n;
      const bool rv = row < N;
      if (packed) {
        const u2 sv = __builtin_bit_cast(
            u2, __builtin_amdgcn_raw_buffer_load_b64(rs, rv ? ((uint32_t)row * G + g0) * 2u : OOB, 0, 0));
        const uint32_t z = bload4(rz, rv ? (uint32_t)row * zrow + 4u * (uint32_t)(g0 / 8) : OOB);
#pragma unroll
        for (int u = 0; u < WU; ++u) {
          sb[t][u] = (uint16_t)((u < 2 ? sv.x : sv.y) >> (16 * (u & 1)));
          zw[t][u] = z;
        }
      } else {
#pragma unroll
        for (int u = 0; u < WU; ++u) {
          const int g = g0 + u;
          const bool gv = rv && g < G;
          sb[t][u] = bload2(rs, gv ? ((uint32_t)row * G + g) * 2u : OOB);
          zw[t][u] = bload4(rz, gv ? (uint32_t)row * zrow + 4u * (uint32_t)(g / 8) : OOB);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < WU; ++u)
#pragma unroll
      for (int t = 0; t < TR; ++t) {
        const uint32_t zq = (zw[t][u] >> (4 * ((g0 + u) % 8))) & 15u;
        const float sc = h2f(sb[t][u]);  // lane l: weight row l % 16 of tile-row t
        if constexpr (MODE == W4A8_PAD) {
          const uint32_t z4 = zq * 0x01010101u;
          const uint2 b0 = codes_minus_z(w[t][u][0], z4), b1 = codes_minus_z(w[t][u][1], z4);
          const uint2 b2 = codes_minus_z(w[t][u][2], z4), b3 = codes_minus_z(w[t][u][3], z4);
          // step s: k 32 kq + 16 s .. + 15 on both sides
          v4i d = {0, 0, 0, 0};
          d = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, x0[u]),
                                                    v4i{(int)b0.x, (int)b0.y, (int)b1.x, (int)b1.y}, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, x1[u]),
                                                    v4i{(int)b2.x, (int)b2.y, (int)b3.x, (int)b3.y}, d, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(sc, (float)d[i], acc[t][i]);
        } else if constexpr (MODE == W4A8_SPLIT) {
          // B: the lane's 32 k of q - z as fp8; A: the same 32 k of the low
          // slices, then of the high slices (16 h): one accumulator adds the
          // two exact partial products (integers below 2^24)
          const v8i b = codes_minus_z_fp8(w[t][u], zq, mg);
          const v8i al = {(int)l0[u][0], (int)l0[u][1], (int)l0[u][2], (int)l0[u][3],
                          (int)l1[u][0], (int)l1[u][1], (int)l1[u][2], (int)l1[u][3]};
          const v8i ah = {(int)x0[u][0], (int)x0[u][1], (int)x0[u][2], (int)x0[u][3],
                          (int)x1[u][0], (int)x1[u][1], (int)x1[u][2], (int)x1[u][3]};
          f4 d = {0.f, 0.f, 0.f, 0.f};
          d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(al, b, d, 0, 0, 0, 0, 0, 0);
          d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ah, b, d, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(sc, d[i], acc[t][i]);
        } else {
          // raw codes on both sides, then the zero-point expansion per group:
          // sum (q - z)(x_q - zx) = sum q x_q - z sum x_q - zx sum q + 128 z zx
          const uint2 b0 = codes_raw(w[t][u][0]), b1 = codes_raw(w[t][u][1]);
          const uint2 b2 = codes_raw(w[t][u][2]), b3 = codes_raw(w[t][u][3]);
          v4i d = {0, 0, 0, 0};
          d = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, x0[u]),
                                                    v4i{(int)b0.x, (int)b0.y, (int)b1.x, (int)b1.y}, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, x1[u]),
                                                    v4i{(int)b2.x, (int)b2.y, (int)b3.x, (int)b3.y}, d, 0, 0, 0);
          // sum of the weight row's 128 codes: the lane's 32 (v_dot8 on the
          // packed nibbles), then the row's four k-quarters
          uint32_t sq = 0u;
#pragma unroll
          for (int e = 0; e < 4; ++e) sq = __builtin_amdgcn_udot8(w[t][u][e], 0x11111111u, sq, false);
          const int sqr = (int)quarter_sum_u(sq);
          const int z = (int)zq;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = d[i] - z * (int)xs[u][i] - zxl[i] * sqr + 128 * z * zxl[i];
            acc[t][i] = fmaf(sc, (float)e, acc[t][i]);
          }
        }
      }
  }
  // lane l holds D[activation row 4 (l / 16) + i][weight row l % 16]
#pragma unroll
  for (int t = 0; t < TR; ++t) reinterpret_cast<f4*>(red)[(wave * TR + t) * 64 + lane] = acc[t];
  __syncthreads();
  for (int e = threadIdx.x; e < 256 * TR; e += blockDim.x) {
    const int i = e & 3, l = (e >> 2) & 63, t = e >> 8;
    const int m = 4 * (l >> 4) + i, col = 16 * (rt0 + t) + (l & 15);
    if (m >= M || col >= N) continue;
    float sum = 0.f;
    for (int w = 0; w < WK; ++w) sum += red[((w * TR + t) * 64 + l) * 4 + i];
    a.y[(size_t)m * N + col] = f2h(a.sx[m] * sum);
  }
}

}  // namespace

size_t w4a8_ws_bytes(int M, int K) { return w4a8_ws_layout(W4A8_PAD, M, K).total; }

// padding: x_q [M, K], s_x [M]; split: 16 h [M, K], l [M, K], s_x [M];
// asymmetric: x_q [M, K], s_x [16], zx [16], sums [K/128][16]; each part
// starting on a 16-byte boundary
W4A8Ws w4a8_ws_layout(int mode, int M, int K) {
  auto up16 = [](size_t v) { return (v + 15) / 16 * 16; };
  const size_t mk = up16((size_t)M * K);
  W4A8Ws l{0, 0, 0, 0, 0, 0};
  if (mode == W4A8_SPLIT) {
    l.xl = mk;
    l.sx = 2 * mk;
    l.total = l.sx + (size_t)M * 4;
  } else if (mode == W4A8_ASYM) {
    l.sx = mk;
    l.zx = l.sx + 64;
    l.xsum = l.zx + 64;
    l.total = l.xsum + (size_t)(K / 128) * 64;
  } else {
    l.sx = mk;
    l.total = l.sx + (size_t)M * 4;
  }
  return l;
}

// Scratch of the entry point that allocates nothing (qgemv_w4a8_noalloc):
// the int8 activations and fp32 row scales of one call, in a file-scope
// device array.  Every GPU the library runs on holds its own copy until the
// process ends; all calls on one GPU share it.  In host code `scratch` names
// a host-side stand-in, never the device memory: host code uses only the
// address hipGetSymbolAddress returns for the current device.
constexpr size_t NOALLOC_SCRATCH_BYTES = W4A8_NOALLOC_MAX_MK + 16 * 4 + 256;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];
static_assert(NOALLOC_SCRATCH_BYTES >= W4A8_NOALLOC_MAX_MK + 15 + 16 * 4, "room for x_q and s_x at M <= 16");

size_t w4a8_noalloc_scratch_bytes() { return NOALLOC_SCRATCH_BYTES; }

// Device address of `scratch` on the calling thread's current device, looked
// up once per device (with that device current) and kept.
hipError_t w4a8_noalloc_scratch(void** ptr) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static void* addr[MAX_DEV] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// waves per workgroup: as the decode VALU engine's one-group chunks (16 for
// long K, 4 on wide layers, else 8), at most one per run of WU groups
int w4a8_waves(int N, int K) {
  const int G = K / 128, nt = (N + 15) / 16;
  const int wk = G >= 96 ? 16 : (nt >= 1024 ? 4 : 8), runs = (G + WU - 1) / WU;
  return wk > runs ? runs : wk;
}

// tile-rows per workgroup: 2 from 9 activation rows on where the grid stays
// wide (384 tile-rows or more), else 1 (8B layers at M = 16: gate+up 25.0 ->
// 23.0 us, qkv 11.0 -> 10.5; at M = 8 and on narrower layers 2 is slower)
int w4a8_tile_rows(int M, int N) { return M > 8 && (N + 15) / 16 >= 384 ? 2 : 1; }

hipError_t launch_gemv_w4a8(const W4A8Args& a, int wk, hipStream_t s) {
  if (wk < 1 || wk > 16) return hipErrorInvalidValue;
  // (the split strategy holds both activation slices of a run in registers:
  // one tile-row per workgroup)
  int tr = a.mode == W4A8_SPLIT ? 1 : w4a8_tile_rows(a.M, a.N);
  if (const char* e = tune_env("QGEMV_W4A8_TR")) tr = std::atoi(e);  // tuning override (1, 2; split: 1)
  if (tr != 1 && tr != 2) return hipErrorInvalidValue;
  const dim3 qg((a.K / 8 + QT - 1) / QT, a.M);
  const int NT = (a.N + 15) / 16;
  const size_t lds = (size_t)wk * tr * 64 * 16;
  const dim3 gg(tr == 2 ? (NT + 1) / 2 : NT), gb(64 * wk);
  switch (a.mode * 10 + tr) {
    case W4A8_PAD * 10 + 1:
      hipLaunchKernelGGL(quant_rows_kernel<W4A8_PAD>, qg, dim3(QT), 0, s, a);
      hipLaunchKernelGGL((gemv_w4a8_kernel<1, W4A8_PAD>), gg, gb, lds, s, a);
      break;
    case W4A8_PAD * 10 + 2:
      hipLaunchKernelGGL(quant_rows_kernel<W4A8_PAD>, qg, dim3(QT), 0, s, a);
      hipLaunchKernelGGL((gemv_w4a8_kernel<2, W4A8_PAD>), gg, gb, lds, s, a);
      break;
    case W4A8_SPLIT * 10 + 1:
      hipLaunchKernelGGL(quant_rows_kernel<W4A8_SPLIT>, qg, dim3(QT), 0, s, a);
      hipLaunchKernelGGL((gemv_w4a8_kernel<1, W4A8_SPLIT>), gg, gb, lds, s, a);
      break;
    case W4A8_ASYM * 10 + 1:
      hipLaunchKernelGGL(quant_rows_kernel<W4A8_ASYM>, qg, dim3(QT), 0, s, a);
      hipLaunchKernelGGL((gemv_w4a8_kernel<1, W4A8_ASYM>), gg, gb, lds, s, a);
      break;
    case W4A8_ASYM * 10 + 2:
      hipLaunchKernelGGL(quant_rows_kernel<W4A8_ASYM>, qg, dim3(QT), 0, s, a);
      hipLaunchKernelGGL((gemv_w4a8_kernel<2, W4A8_ASYM>), gg, gb, lds, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qg
