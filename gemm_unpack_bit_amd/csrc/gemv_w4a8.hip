// W4A8 GEMV with the padding strategy (ADAngel review, DPR: padding extends
// the low-bit weight to the activation width), on the int8 matrix cores:
//
//   x_q[m, k] = rint(x[m, k] / s_x[m]) clamped to [-127, 127],
//   s_x[m] = max_k |x[m, k]| / 127                        (fp32)
//   y[m, n]   = s_x[m] * sum_g s_w[n, g] * sum_{k in g} (q[n, k] - z[n, g]) x_q[m, k]
//
// Two kernels on the caller's stream:
//  * quant_rows_kernel: writes x_q (int8) and s_x (fp32) to the caller's
//    workspace; fp32 correctly rounded division and round-to-nearest-even,
//    so x_q is the exact integer the definition gives.  Each workgroup takes
//    2048 k of one row: it reads the whole row for the max (exact in any
//    order, so every workgroup of the row finds the same s_x) and quantizes
//    its own part, which it already holds in registers.
//  * gemv_w4a8_kernel<TR>: a workgroup owns TR (1 or 2) 16-row tile-rows of
//    the 4-bit tiled device layout; its waves take runs of WU quant groups
//    round-robin, issuing all of a run's loads before its MFMAs.  A lane's
//    4 code words hold its row's 32 k of the group; two byte permutes put a
//    word's 8 codes in k order, one or/subtract/xor turns them into the
//    signed bytes q - z (no borrow between bytes), and 16 of them are the B
//    operand of v_mfma_i32_16x16x64_i8 (A: the same 16 k of 16 activation
//    rows).  The int32 group sums are exact; each is scaled by the lane's
//    row scale, the waves are added in a fixed order through LDS, and the
//    row's activation scale is applied last.  Deterministic.
#include <cstdlib>
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

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

// grid: (K / 2048 rounded up, M)
__global__ void __launch_bounds__(QT) quant_rows_kernel(W4A8Args a) {
  __shared__ float wmax[QT / 64];
  const int m = blockIdx.y, K = a.K, tid = threadIdx.x;
  const int np = K / 8;                       // 16-byte pieces of the row
  const int mine = blockIdx.x * QT + tid;     // the piece this thread quantizes
  const rsrc_t rx = make_rsrc(a.x + (size_t)m * K, (uint32_t)K * 2u);
  u4 own = u4{0u, 0u, 0u, 0u};
  float amax = 0.f;
  for (int base = tid; base < np; base += QT * QU) {
    u4 v[QU];
#pragma unroll
    for (int j = 0; j < QU; ++j) {
      const int p = base + QT * j;
      v[j] = bload16(rx, p < np ? 16u * p : OOB);  // (past the row: zeros)
    }
#pragma unroll
    for (int j = 0; j < QU; ++j) {
      amax = fmaxf(amax, h8_absmax(v[j]));
      if (base + QT * j == mine) own = v[j];
    }
  }
  // max over the workgroup (exact, any order)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = amax;
  __syncthreads();
  amax = 0.f;
#pragma unroll
  for (int w = 0; w < QT / 64; ++w) amax = fmaxf(amax, wmax[w]);
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
    *reinterpret_cast<uint2*>(a.xq + (size_t)m * K + 8 * (size_t)mine) = uint2{lo, hi};
  }
  if (blockIdx.x == 0 && tid == 0) a.sx[m] = s;
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

constexpr int WU = 4;  // quant groups per wave whose loads are in flight together

// TR tile-rows per workgroup (1, 2): with 2, each A fragment loaded from L2
// serves both tile-rows, halving the activation reads (they reach twice the
// weight bytes at M = 16).
template <int TR>
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
  // A: activation row n (rows past M read zeros), the lane's 32 k of a group
  const uint32_t xo = n < M ? (uint32_t)n * K + 32u * kq : OOB;
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
    u4 w[TR][WU], x0[WU], x1[WU];
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
        const uint32_t z4 = ((zw[t][u] >> (4 * ((g0 + u) % 8))) & 15u) * 0x01010101u;
        const uint2 b0 = codes_minus_z(w[t][u][0], z4), b1 = codes_minus_z(w[t][u][1], z4);
        const uint2 b2 = codes_minus_z(w[t][u][2], z4), b3 = codes_minus_z(w[t][u][3], z4);
        // step s: k 32 kq + 16 s .. + 15 on both sides
        v4i d = {0, 0, 0, 0};
        d = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, x0[u]),
                                                  v4i{(int)b0.x, (int)b0.y, (int)b1.x, (int)b1.y}, d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, x1[u]),
                                                  v4i{(int)b2.x, (int)b2.y, (int)b3.x, (int)b3.y}, d, 0, 0, 0);
        const float sc = h2f(sb[t][u]);  // lane l: weight row l % 16 of tile-row t
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] = fmaf(sc, (float)d[i], acc[t][i]);
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

size_t w4a8_ws_bytes(int M, int K) { return ((size_t)M * K + 15) / 16 * 16 + (size_t)M * 4; }

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
  int tr = w4a8_tile_rows(a.M, a.N);
  if (const char* e = tune_env("QGEMV_W4A8_TR")) tr = std::atoi(e);  // tuning override (1, 2)
  if (tr != 1 && tr != 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((a.K / 8 + QT - 1) / QT, a.M), dim3(QT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int NT = (a.N + 15) / 16;
  const size_t lds = (size_t)wk * tr * 64 * 16;
  if (tr == 2)
    hipLaunchKernelGGL(gemv_w4a8_kernel<2>, dim3((NT + 1) / 2), dim3(64 * wk), lds, s, a);
  else
    hipLaunchKernelGGL(gemv_w4a8_kernel<1>, dim3(NT), dim3(64 * wk), lds, s, a);
  return hipGetLastError();
}

}  // namespace qg
