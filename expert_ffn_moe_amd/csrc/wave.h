// Wavefront (64-lane) primitives for gfx950: DPP butterflies inside a row of 16 lanes,
// cross-lane permutes across rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// DPP control words (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  uint32_t lo = dpp_u32<CTRL>((uint32_t)v);
  uint32_t hi = dpp_u32<CTRL>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// All-reduce max over the 64 lanes of a wavefront (all lanes must be active).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<kDppQuadXor1>(v));
  v = max_u64(v, dpp_u64<kDppQuadXor2>(v));
  v = max_u64(v, dpp_u64<kDppRowHalfMirror>(v));
  v = max_u64(v, dpp_u64<kDppRowMirror>(v));
  v = max_u64(v, shfl_xor_u64(v, 16));
  v = max_u64(v, shfl_xor_u64(v, 32));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

}  // namespace moe
