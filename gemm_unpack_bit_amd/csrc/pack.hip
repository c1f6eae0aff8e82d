// Bit packing on the device: [rows, cols] one-code-per-byte <-> packed words.
//
// Plain layout: row-major rows of ceil(cols*b/32) words; word j of a row holds
// columns [j*P, (j+1)*P) (P = 32/b), field f holding column j*P + f.
//
// Device layout (the weights of every compute entry point; cols % 128 == 0):
// tiles of 16 rows x 128 columns (rows padded with code 0 to a multiple of
// 16).  Tile (rt, g) starts at word (rt*G + g) * 64*b (G = cols/128).  Inside
// it, lane l in [0, 64) owns row 16*rt + l%16 and the 32 columns
// [128*g + 32*(l/16), +32) as b words; word i of lane l sits at tile word
// (i/4)*256 + l*min(b,4) + i%4 and covers columns 128*g + 32*(l/16) + P*i +
// [0, P) with field f holding offset 2f (f < P/2) or 2(f - P/2) + 1
// (f >= P/2): the two 16-bit halves of a word carry consecutive columns.
//
// Row-block layout (layout 2, 8-bit codes only; the codebook variant's code
// format): tiles of 64 rows x 16 columns (1 KB), tile (rb, cb) at byte
// (rb * ceil(cols/16) + cb) * 1024, byte 16 l + i holding column 16 cb + i of
// row 64 rb + l.  A wave-wide 16-byte load of one tile gives lane l 16
// consecutive codes of its own row.  Rows and columns past the matrix are 0.
#include "common.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

__device__ int g_pack_bad_code;  // set when a code does not fit in b bits

// column offset (inside its word) held by field f of a device word
template <int BITS>
__device__ __forceinline__ int field_col(int f) {
  constexpr int HALF = 16 / BITS;
  return f < HALF ? 2 * f : 2 * (f - HALF) + 1;
}

// (row, first column) of device word `idx`
template <int BITS>
__device__ __forceinline__ void tile_word_pos(size_t idx, int G, int& row, int& col) {
  constexpr int TW = 64 * BITS;            // words per tile
  constexpr int LW = BITS < 4 ? BITS : 4;  // words per lane per 1 KB half
  const size_t tile = idx / TW;
  const int within = (int)(idx % TW);
  const int h = within / 256, rem = within % 256;
  const int lane = rem / LW, e = rem % LW;
  const int i = 4 * h + e;
  const int rt = (int)(tile / G), g = (int)(tile % G);
  row = 16 * rt + lane % 16;
  col = 128 * g + 32 * (lane / 16) + (32 / BITS) * i;
}

template <int BITS, bool TILED>
__global__ void pack_kernel(const uint8_t* __restrict__ codes, uint32_t* __restrict__ packed, int rows,
                            int cols, size_t nwords) {
  constexpr int PER = 32 / BITS;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= nwords) return;
  int r, c0;
  if constexpr (TILED) {
    tile_word_pos<BITS>(idx, cols / 128, r, c0);
  } else {
    const int wpr = (cols * BITS + 31) / 32;
    r = (int)(idx / wpr);
    c0 = (int)(idx % wpr) * PER;
  }
  uint32_t word = 0;
  bool bad = false;
  if (r < rows) {
    const uint8_t* src = codes + (size_t)r * cols;
#pragma unroll
    for (int f = 0; f < PER; ++f) {
      const int c = c0 + (TILED ? field_col<BITS>(f) : f);
      if (c < cols) {
        const uint32_t q = src[c];
        bad |= q >> BITS;
        word |= (q & ((1u << BITS) - 1u)) << (BITS * f);
      }
    }
  }
  if (bad) g_pack_bad_code = 1;
  packed[idx] = word;
}

__global__ void pack_rows64_kernel(const uint8_t* __restrict__ codes, uint32_t* __restrict__ packed, int rows,
                                   int cols, size_t nwords) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= nwords) return;
  const int ncb = (cols + 15) / 16;
  const size_t tile = idx / 256;
  const int within = (int)(idx % 256);
  const int l = within / 4, d = within % 4;
  const int r = (int)(tile / ncb) * 64 + l;
  const int c0 = (int)(tile % ncb) * 16 + 4 * d;
  uint32_t word = 0;
  if (r < rows) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
      if (c0 + f < cols) word |= (uint32_t)codes[(size_t)r * cols + c0 + f] << (8 * f);
  }
  packed[idx] = word;
}

__global__ void unpack_rows64_kernel(const uint32_t* __restrict__ packed, uint8_t* __restrict__ codes, int rows,
                                     int cols) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)rows * cols) return;
  const int r = (int)(idx / cols), c = (int)(idx % cols);
  const int ncb = (cols + 15) / 16;
  const size_t byte = ((size_t)(r / 64) * ncb + c / 16) * 1024 + 16 * (r % 64) + c % 16;
  codes[idx] = (uint8_t)(packed[byte / 4] >> (8 * (byte % 4)));
}

template <int BITS, bool TILED>
__global__ void unpack_kernel(const uint32_t* __restrict__ packed, uint8_t* __restrict__ codes, int rows,
                              int cols) {
  constexpr int PER = 32 / BITS;
  constexpr int HALF = PER / 2;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)rows * cols) return;
  const int r = (int)(idx / cols), c = (int)(idx % cols);
  size_t word;
  int f;
  if constexpr (TILED) {
    constexpr int LW = BITS < 4 ? BITS : 4;
    const int G = cols / 128, g = c / 128, cq = (c % 128) / 32, o = c % 32;
    const int i = o / PER, oi = o % PER;
    const int lane = 16 * cq + r % 16;
    word = ((size_t)(r / 16) * G + g) * (64 * BITS) + (i / 4) * 256 + lane * LW + i % 4;
    f = (oi & 1) ? HALF + oi / 2 : oi / 2;
  } else {
    word = (size_t)r * ((cols * BITS + 31) / 32) + c / PER;
    f = c % PER;
  }
  codes[idx] = (uint8_t)((packed[word] >> (BITS * f)) & ((1u << BITS) - 1u));
}

__global__ void clear_flag_kernel() { g_pack_bad_code = 0; }

template <bool TILED>
hipError_t pack_l(int bits, int rows, int cols, const uint8_t* codes, uint32_t* packed, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, s);
  if (n == 0) return hipGetLastError();
  const dim3 grid((unsigned)((n + 255) / 256));
  switch (bits) {
    case 2: hipLaunchKernelGGL((pack_kernel<2, TILED>), grid, dim3(256), 0, s, codes, packed, rows, cols, n); break;
    case 4: hipLaunchKernelGGL((pack_kernel<4, TILED>), grid, dim3(256), 0, s, codes, packed, rows, cols, n); break;
    case 8: hipLaunchKernelGGL((pack_kernel<8, TILED>), grid, dim3(256), 0, s, codes, packed, rows, cols, n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool TILED>
hipError_t unpack_l(int bits, int rows, int cols, const uint32_t* packed, uint8_t* codes, hipStream_t s) {
  const size_t n = (size_t)rows * cols;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  switch (bits) {
    case 2: hipLaunchKernelGGL((unpack_kernel<2, TILED>), grid, dim3(256), 0, s, packed, codes, rows, cols); break;
    case 4: hipLaunchKernelGGL((unpack_kernel<4, TILED>), grid, dim3(256), 0, s, packed, codes, rows, cols); break;
    case 8: hipLaunchKernelGGL((unpack_kernel<8, TILED>), grid, dim3(256), 0, s, packed, codes, rows, cols); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t packed_words(int bits, int layout, int rows, int cols) {
  if (layout == 2) return bits == 8 ? (size_t)((rows + 63) / 64) * 64 * (size_t)((cols + 15) / 16) * 4 : 0;
  if (layout) return (size_t)((rows + 15) / 16) * 16 * (size_t)cols * bits / 32;
  return (size_t)rows * (size_t)(((long)cols * bits + 31) / 32);
}

hipError_t launch_pack(int bits, int layout, int rows, int cols, const uint8_t* codes, uint32_t* packed,
                       hipStream_t s) {
  const size_t n = packed_words(bits, layout, rows, cols);
  if (layout == 2) {  // 8-bit codes: every byte value is a valid code
    hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, s);
    if (n) hipLaunchKernelGGL(pack_rows64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, packed,
                              rows, cols, n);
    return hipGetLastError();
  }
  return layout ? pack_l<true>(bits, rows, cols, codes, packed, n, s)
                : pack_l<false>(bits, rows, cols, codes, packed, n, s);
}

hipError_t launch_unpack(int bits, int layout, int rows, int cols, const uint32_t* packed, uint8_t* codes,
                         hipStream_t s) {
  if (layout == 2) {
    const size_t n = (size_t)rows * cols;
    if (n) hipLaunchKernelGGL(unpack_rows64_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, packed, codes,
                              rows, cols);
    return hipGetLastError();
  }
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
