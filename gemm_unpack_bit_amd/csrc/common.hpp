// Device-side helpers shared by the qgemv kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// fp32 += a.lo*b.lo + a.hi*b.hi   (v_dot2_f32_f16)
__device__ __forceinline__ float dot2(h2 a, h2 b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

// a.lo*b.lo + a.hi*b.hi into a fresh fp32: the VOP3 form with an
// inline-constant 0 accumulator (the builtin with a 0 accumulator becomes
// the tied-accumulator form and a v_mov of 0 before it)
__device__ __forceinline__ float dot2_first(h2 a, h2 b) {
  float d;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

__device__ __forceinline__ h2 fma2(h2 a, h2 b, h2 c) { return __builtin_elementwise_fma(a, b, c); }

__device__ __forceinline__ float h2f(uint16_t bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}
__device__ __forceinline__ uint16_t f2h(float v) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Cross-lane move through DPP; lanes masked off by ROW_MASK read 0.
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, BANK_MASK, false));
}

enum : int {
  DPP_QP_XOR1 = 0xB1,   // quad_perm [1,0,3,2]
  DPP_QP_XOR2 = 0x4E,   // quad_perm [2,3,0,1]
  DPP_ROR4 = 0x124,     // row_ror:4
  DPP_ROR8 = 0x128,     // row_ror:8
  DPP_BCAST15 = 0x142,  // row_bcast:15
  DPP_BCAST31 = 0x143,  // row_bcast:31
};

// Sum over each group of LANES consecutive lanes (LANES in {16, 32, 64}).
// The sum ends up in the last lane of each group (for 16 it is in every lane).
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<DPP_QP_XOR1>(v);
  v += dpp<DPP_QP_XOR2>(v);
  v += dpp<DPP_ROR4>(v);
  v += dpp<DPP_ROR8>(v);
  if constexpr (LANES >= 32) v += dpp<DPP_BCAST15, 0xA>(v);
  if constexpr (LANES >= 64) v += dpp<DPP_BCAST31, 0xC>(v);
  return v;
}

// d = (a & mask) | c as one VALU op.  The mask goes through an SGPR and c
// through a VGPR because gfx9-family VOP3 encodings take no literal constant.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(mask), "v"(c));
  return d;
}

// A VGPR holding the fp16x2 bit pattern (1024, 1024); opaque to constant
// folding so that and_or() can take it as its VGPR operand.
__device__ __forceinline__ uint32_t magic1024x2() {
  uint32_t v;
  asm("v_mov_b32 %0, 0x64006400" : "=v"(v));
  return v;
}

// Sum of the values held by lanes n, n + 16, n + 32, n + 48 of a wave,
// returned in all four lanes, in the fixed order (q0 + q2) + (q1 + q3)
// (gfx950 permlane swaps; every lane of the wave must take part).
__device__ __forceinline__ float quarter_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t su = __float_as_uint(s);
  const auto b = __builtin_amdgcn_permlane16_swap(su, su, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over waves w < WK (WK <= 16) of per-wave partials red[w * OUT + o],
// OUT a multiple of 16, after a barrier.  Output o is summed by the four lanes
// l, l + 16, l + 32, l + 48 of one wave -- lane quarter q takes waves q, q + 4,
// q + 8, q + 12, all reads issued together -- then across the quarters: a
// fixed order, so the result is deterministic.  store(o, sum) runs once per
// output, in lane l < 16 of the wave that summed it.
template <typename F>
__device__ __forceinline__ void reduce_waves(const float* red, int OUT, int WK, F&& store) {
  const int lane = threadIdx.x & 63, q = lane >> 4;
  const int nw = blockDim.x >> 6;
  for (int o0 = (threadIdx.x >> 6) * 16; o0 < OUT; o0 += nw * 16) {  // wave-uniform
    const int o = o0 + (lane & 15);
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int w = q + 4 * i;
      v[i] = red[(w < WK ? w : 0) * OUT + o];
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) sum = q + 4 * i < WK ? sum + v[i] : sum;
    sum = quarter_sum(sum);
    if (q == 0) store(o, sum);
  }
}

// i / d for 0 <= i < 2^22 and 1 <= d < 2^22, exact, with inv = 1.0f / d:
// the float estimate is off by at most one below 2^23, and one correction
// each way fixes it (a few full-rate VALU ops instead of an integer
// division sequence).
__device__ __forceinline__ int div_small(int i, int d, float inv) {
  int q = (int)((float)i * inv);
  q -= __mul24(q, d) > i ? 1 : 0;
  q += __mul24(q + 1, d) <= i ? 1 : 0;
  return q;
}

// Workgroup barrier that orders LDS only: each wave waits for its own LDS
// operations (lgkmcnt 0) and meets the others at s_barrier, while its global
// loads stay in flight.  __syncthreads() would also wait for every vector
// memory load (prefetches included), draining a software pipeline.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Raw buffer resource over [base, base + bytes): loads at byte offsets >= bytes
// return 0 without touching memory (hardware bounds check), so ragged edges
// need no branches.  Word 3 = 0x00020000 selects 32-bit data format.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int CPOL_NT = 2;             // non-temporal (streaming) cache policy
constexpr uint32_t OOB = 0x80000000u;  // an offset past every buffer we use

// `off` is the per-lane byte offset (VGPR); `soff` a wave-uniform byte offset
// that goes in the instruction's scalar offset (SGPR), costing no VALU.
template <int CPOL = 0>
__device__ __forceinline__ u4 bload16(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, CPOL);
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
}
__device__ __forceinline__ uint16_t bload2(rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
}

// Streaming (non-temporal) 16-byte load: weights are read once per call.
__device__ __forceinline__ u4 load_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
}

}  // namespace qg
