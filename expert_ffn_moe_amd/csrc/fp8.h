// FP8 (OCP E4M3) helpers shared by the quantisation kernels and the FP8 GEMM epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kQBlock = 32;  // elements per UE8M0 scale block

// Scale exponent of a block with absolute maximum amax: the smallest integer e with
// amax <= 448 * 2^e (0 for amax == 0), clamped to the E8M0 range.  With
// amax = m * 2^x, m in [0.5, 1) and 448 = 0.875 * 2^9: e = x - 9 + (m > 0.875).
__device__ __forceinline__ int ue8m0_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int x;
  const float m = frexpf(amax, &x);
  const int e = x - 9 + (m > 0.875f ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Four values scaled by 2^s (exact) and rounded to E4M3 (nearest, ties to even) by the
// hardware conversion, packed little-endian into one word.
__device__ __forceinline__ uint32_t pack_fp8x4(const float* f, int s) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[0], s), ldexpf(f[1], s), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[2], s), ldexpf(f[3], s), w, true);
  return (uint32_t)w;
}

}  // namespace moe
