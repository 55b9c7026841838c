// Combine (LightLLM PR #1687 walkthrough, "Synchronous prefill and decode execution":
// expert outputs are reduced into dense token output):
//   y[t] = sum over slots j in order, skipping dropped ones, of w[t,j] * yp[slot_to_row[t,j]]
// fp32 accumulation in slot order, one token per block: deterministic, no atomics.
#include "bf16.h"
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint4* __restrict__ yp,
                                                           const float* __restrict__ w,
                                                           const int32_t* __restrict__ s2r,
                                                           int k, int nvec,
                                                           uint4* __restrict__ y) {
  __shared__ int rows[32];
  __shared__ float wt[32];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = s2r[(size_t)t * k + threadIdx.x];
    wt[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < k; ++j) {
      const int r = rows[j];
      if (r < 0) continue;
      float f[8];
      unpack8(yp[(size_t)r * nvec + v], f);
      const float wj = wt[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, f[i], acc[i]);
    }
    y[(size_t)t * nvec + v] = pack8(acc);
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float4* __restrict__ yp,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ s2r,
                                                          int k, int nvec,
                                                          float4* __restrict__ y) {
  __shared__ int rows[32];
  __shared__ float wt[32];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = s2r[(size_t)t * k + threadIdx.x];
    wt[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int r = rows[j];
      if (r < 0) continue;
      const float4 f = yp[(size_t)r * nvec + v];
      const float wj = wt[j];
      acc.x = __builtin_fmaf(wj, f.x, acc.x);
      acc.y = __builtin_fmaf(wj, f.y, acc.y);
      acc.z = __builtin_fmaf(wj, f.z, acc.z);
      acc.w = __builtin_fmaf(wj, f.w, acc.w);
    }
    y[(size_t)t * nvec + v] = acc;
  }
}

}  // namespace

hipError_t launch_combine(const moe_problem& p, const void* yp, const float* w,
                          const int32_t* slot_to_row, void* y, hipStream_t s) {
  if (p.act_dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_bf16_kernel, dim3(p.T), dim3(256), 0, s, (const uint4*)yp, w,
                       slot_to_row, p.k, p.H / 8, (uint4*)y);
  else
    hipLaunchKernelGGL(combine_f32_kernel, dim3(p.T), dim3(256), 0, s, (const float4*)yp, w,
                       slot_to_row, p.k, p.H / 4, (float4*)y);
  return hipGetLastError();
}

}  // namespace moe
