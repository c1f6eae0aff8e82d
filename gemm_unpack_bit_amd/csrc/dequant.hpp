// Unpack of device-packed b-bit codes to exact fp16 (q - z) pairs, shared by
// the VALU and MFMA kernels.
//
// Each b-bit field is OR-ed into the mantissa of fp16 1024.0 (bits 0x6400):
// a field at bit offset 2c of a 16-bit half yields exactly 1024 + 4^c q.  One
// packed fp16 op per pair then gives q - z exactly:
// (1024 + 4^c q) * 4^-c - (1024 * 4^-c + z).  In the device layout fields f and
// f + P/2 of a word hold consecutive k, so pair i of a word is (k + 2i, k + 2i + 1).
#pragma once

#include "common.hpp"

namespace qg {

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

// ---------------------------------------------------------------------------
// streaming a lane's share of one 16 x 128 tile of the device layout
// ---------------------------------------------------------------------------
// One lane's codes of one tile: 32 codes = b words, in <= 2 loads.
template <int BITS>
struct LaneCodes {
  uint32_t w[BITS];
  // `off` = lane offset inside the tile (VGPR) or OOB, `soff` = tile offset (SGPR)
  __device__ __forceinline__ void load(rsrc_t r, uint32_t off, uint32_t soff) {
    if constexpr (BITS == 2) {
      const u2 v = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, CPOL_NT));
      w[0] = v[0];
      w[1] = v[1];
    } else {
#pragma unroll
      for (int h = 0; h < BITS / 4; ++h) {
        const u4 v = bload16<CPOL_NT>(r, off + 1024u * h, soff);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[4 * h + e] = v[e];
      }
    }
  }
};

// Lane byte offset inside a tile (its first word).
template <int BITS>
__device__ __forceinline__ uint32_t lane_off(int lane) {
  return (uint32_t)lane * 4u * (BITS < 4 ? BITS : 4);
}

}  // namespace qg
