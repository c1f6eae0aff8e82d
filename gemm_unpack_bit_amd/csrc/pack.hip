// Bit packing on the device: [rows, cols] one-code-per-byte <-> rows of
// ceil(cols*b/32) uint32 words; word j holds columns [j*P, (j+1)*P), P = 32/b.
// Plain layout: field f holds column j*P + f.  Device layout: field f holds
// column j*P + 2f (f < P/2) or j*P + 2(f - P/2) + 1 (f >= P/2).
#include "common.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

__device__ int g_pack_bad_code;  // set when a code does not fit in b bits

// column offset (inside its word) held by field f
template <int BITS, bool DEVICE>
__device__ __forceinline__ int field_col(int f) {
  constexpr int HALF = 16 / BITS;
  if constexpr (DEVICE) return f < HALF ? 2 * f : 2 * (f - HALF) + 1;
  return f;
}

template <int BITS, bool DEVICE>
__global__ void pack_kernel(const uint8_t* __restrict__ codes, uint32_t* __restrict__ packed, int rows,
                            int cols, int wpr) {
  constexpr int PER = 32 / BITS;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)rows * wpr) return;
  const int r = (int)(idx / wpr), j = (int)(idx % wpr);
  const uint8_t* src = codes + (size_t)r * cols;
  uint32_t word = 0;
  bool bad = false;
#pragma unroll
  for (int f = 0; f < PER; ++f) {
    const int c = j * PER + field_col<BITS, DEVICE>(f);
    if (c < cols) {
      const uint32_t q = src[c];
      bad |= q >> BITS;
      word |= (q & ((1u << BITS) - 1u)) << (BITS * f);
    }
  }
  if (bad) g_pack_bad_code = 1;
  packed[idx] = word;
}

template <int BITS, bool DEVICE>
__global__ void unpack_kernel(const uint32_t* __restrict__ packed, uint8_t* __restrict__ codes, int rows,
                              int cols, int wpr) {
  constexpr int PER = 32 / BITS;
  constexpr int HALF = PER / 2;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)rows * cols) return;
  const int r = (int)(idx / cols), c = (int)(idx % cols);
  const uint32_t w = packed[(size_t)r * wpr + c / PER];
  const int o = c % PER;
  const int f = DEVICE ? ((o & 1) ? HALF + o / 2 : o / 2) : o;
  codes[idx] = (uint8_t)((w >> (BITS * f)) & ((1u << BITS) - 1u));
}

__global__ void clear_flag_kernel() { g_pack_bad_code = 0; }

template <bool DEVICE>
hipError_t pack_l(int bits, int rows, int cols, const uint8_t* codes, uint32_t* packed, hipStream_t s) {
  const int wpr = (cols * bits + 31) / 32;
  const size_t n = (size_t)rows * wpr;
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, s);
  if (n == 0) return hipGetLastError();
  const dim3 grid((unsigned)((n + 255) / 256));
  switch (bits) {
    case 2: hipLaunchKernelGGL((pack_kernel<2, DEVICE>), grid, dim3(256), 0, s, codes, packed, rows, cols, wpr); break;
    case 4: hipLaunchKernelGGL((pack_kernel<4, DEVICE>), grid, dim3(256), 0, s, codes, packed, rows, cols, wpr); break;
    case 8: hipLaunchKernelGGL((pack_kernel<8, DEVICE>), grid, dim3(256), 0, s, codes, packed, rows, cols, wpr); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool DEVICE>
hipError_t unpack_l(int bits, int rows, int cols, const uint32_t* packed, uint8_t* codes, hipStream_t s) {
  const int wpr = (cols * bits + 31) / 32;
  const size_t n = (size_t)rows * cols;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  switch (bits) {
    case 2: hipLaunchKernelGGL((unpack_kernel<2, DEVICE>), grid, dim3(256), 0, s, packed, codes, rows, cols, wpr); break;
    case 4: hipLaunchKernelGGL((unpack_kernel<4, DEVICE>), grid, dim3(256), 0, s, packed, codes, rows, cols, wpr); break;
    case 8: hipLaunchKernelGGL((unpack_kernel<8, DEVICE>), grid, dim3(256), 0, s, packed, codes, rows, cols, wpr); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(int bits, int layout, int rows, int cols, const uint8_t* codes, uint32_t* packed,
                       hipStream_t s) {
  return layout ? pack_l<true>(bits, rows, cols, codes, packed, s) : pack_l<false>(bits, rows, cols, codes, packed, s);
}

hipError_t launch_unpack(int bits, int layout, int rows, int cols, const uint32_t* packed, uint8_t* codes,
                         hipStream_t s) {
  return layout ? unpack_l<true>(bits, rows, cols, packed, codes, s)
                : unpack_l<false>(bits, rows, cols, packed, codes, s);
}

hipError_t pack_error_flag(int* flag, hipStream_t s) {
  hipError_t e = hipMemcpyFromSymbolAsync(flag, HIP_SYMBOL(g_pack_bad_code), sizeof(int), 0,
                                          hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

}  // namespace qg
