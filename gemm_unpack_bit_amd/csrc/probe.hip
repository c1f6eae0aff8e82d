// Streaming-read probe: the achievable HBM read bandwidth that the GEMV
// kernels are measured against.  Reads every 16-byte unit of a device buffer
// once, with the load the weight streams use (16-byte per lane, a wave-wide
// load one contiguous 1 KB burst, non-temporal), and writes nothing unless
// the XOR of the data equals an improbable pattern (so the loads cannot be
// removed).  Grid-stride over the buffer with U loads in flight per lane.
#include "common.hpp"
#include "kernels.hpp"

namespace qg {
namespace {

constexpr int U = 8;

__global__ void __launch_bounds__(1024) stream_read_kernel(const u4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t nth = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  u4 acc = u4{0u, 0u, 0u, 0u};
  for (; i + (U - 1) * nth < n16; i += U * nth) {
    u4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * nth);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n16; i += nth) acc ^= __builtin_nontemporal_load(src + i);
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u && acc[2] == 0xF39CC060u && acc[3] == 0x5CEDC834u)
    sink[0] = acc[0] ^ acc[1];
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, int threads,
                              hipStream_t s) {
  if (workgroups < 1 || threads < 64 || threads > 1024 || threads % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(workgroups), dim3(threads), 0, s, reinterpret_cast<const u4*>(src),
                     bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace qg
