// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

struct UniformArgs {
  int bits, M, N, K;
  const uint16_t* x;
  const uint32_t* wq;
  const uint16_t* scales;
  const uint32_t* zeros;
  uint16_t* y;
};

// VALU GEMV launch shape: MT = x rows per pass (1, 2 or 4); RI = weight rows
// per wave-wide load (1, 2 or 4); NV = 16-byte code vectors per lane and row
// (1 or 2); U = row groups per pipeline stage (2 or 4); WK = waves per
// workgroup splitting K; RB = rows per workgroup (multiple of RI * U).
struct ValuCfg {
  int mt, ri, wk, rb, nv, u;
};

ValuCfg pick_valu(int bits, int M, int N, int K);
hipError_t launch_gemv_valu(const UniformArgs& a, const ValuCfg& c, hipStream_t s);

// bit packing (layout: 0 plain, 1 device)
hipError_t launch_pack(int bits, int layout, int rows, int cols, const uint8_t* codes, uint32_t* packed,
                       hipStream_t s);
hipError_t launch_unpack(int bits, int layout, int rows, int cols, const uint32_t* packed, uint8_t* codes,
                         hipStream_t s);
// reads and clears the pack kernel's out-of-range flag (synchronizes s)
hipError_t pack_error_flag(int* flag, hipStream_t s);

}  // namespace qg
