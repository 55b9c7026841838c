// Combine (LightLLM PR #1687 walkthrough, "Synchronous prefill and decode execution":
// expert outputs are reduced into dense token output):
//   y[t] = sum over slots j in order, skipping dropped ones, of w[t,j] * yp[slot_to_row[t,j]]
// fp32 accumulation in slot order, one token per block: deterministic, no atomics.  With a
// shared expert (PR body: the combine adds the shared expert's output), its row for the
// token is added last, before the one rounding.
#include "bf16.h"
#include "moe_internal.h"

namespace moe {
namespace {

// KMAX > 0: k <= KMAX, the k row loads of a vector are issued together before any of them
// is used (the slot loop unrolled); KMAX = 0: any k, one slot at a time.
template <int KMAX>
__global__ __launch_bounds__(256) void combine_bf16_kernel(const uint4* __restrict__ yp,
                                                           const float* __restrict__ w,
                                                           const int32_t* __restrict__ s2r,
                                                           int k, int nvec,
                                                           const uint4* __restrict__ shared,
                                                           uint4* __restrict__ y) {
  __shared__ int rows[32];
  __shared__ float wt[32];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = s2r[(size_t)t * k + threadIdx.x];
    wt[threadIdx.x] = w ? w[(size_t)t * k + threadIdx.x] : 1.0f;  // NULL: unit weights
  }
  __syncthreads();
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (KMAX > 0) {
      uint4 rv[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < k && rows[j] >= 0) rv[j] = yp[(size_t)rows[j] * nvec + v];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) {
        if (j < k && rows[j] >= 0) {  // block-uniform
          float f[8];
          unpack8(rv[j], f);
          const float wj = wt[j];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, f[i], acc[i]);
        }
      }
    } else {
      for (int j = 0; j < k; ++j) {
        const int r = rows[j];
        if (r < 0) continue;
        float f[8];
        unpack8(yp[(size_t)r * nvec + v], f);
        const float wj = wt[j];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, f[i], acc[i]);
      }
    }
    if (shared) {
      float f[8];
      unpack8(shared[(size_t)t * nvec + v], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = acc[i] + f[i];
    }
    y[(size_t)t * nvec + v] = pack8(acc);
  }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float4* __restrict__ yp,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ s2r,
                                                          int k, int nvec,
                                                          const float4* __restrict__ shared,
                                                          float4* __restrict__ y) {
  __shared__ int rows[32];
  __shared__ float wt[32];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = s2r[(size_t)t * k + threadIdx.x];
    wt[threadIdx.x] = w ? w[(size_t)t * k + threadIdx.x] : 1.0f;  // NULL: unit weights
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
    if (shared) {
      const float4 f = shared[(size_t)t * nvec + v];
      acc.x = acc.x + f.x;
      acc.y = acc.y + f.y;
      acc.z = acc.z + f.z;
      acc.w = acc.w + f.w;
    }
    y[(size_t)t * nvec + v] = acc;
  }
}

// offsets of a one-expert layout of n rows: {0, n}
__global__ void one_expert_offsets_kernel(int32_t* off, int n) {
  if (threadIdx.x < 2) off[threadIdx.x] = threadIdx.x ? n : 0;
}

}  // namespace

hipError_t launch_combine(const moe_problem& p, const void* yp, const float* w,
                          const int32_t* slot_to_row, const void* shared, void* y,
                          hipStream_t s) {
  if (p.act_dtype == MOE_F32)
    hipLaunchKernelGGL(combine_f32_kernel, dim3(p.T), dim3(256), 0, s, (const float4*)yp, w,
                       slot_to_row, p.k, p.H / 4, (const float4*)shared, (float4*)y);
  else if (p.k <= 4)
    hipLaunchKernelGGL(combine_bf16_kernel<4>, dim3(p.T), dim3(256), 0, s, (const uint4*)yp, w,
                       slot_to_row, p.k, p.H / 8, (const uint4*)shared, (uint4*)y);
  else if (p.k <= 8)
    hipLaunchKernelGGL(combine_bf16_kernel<8>, dim3(p.T), dim3(256), 0, s, (const uint4*)yp, w,
                       slot_to_row, p.k, p.H / 8, (const uint4*)shared, (uint4*)y);
  else
    hipLaunchKernelGGL(combine_bf16_kernel<0>, dim3(p.T), dim3(256), 0, s, (const uint4*)yp, w,
                       slot_to_row, p.k, p.H / 8, (const uint4*)shared, (uint4*)y);
  return hipGetLastError();
}

hipError_t launch_one_expert_offsets(int32_t* off, int n, hipStream_t s) {
  hipLaunchKernelGGL(one_expert_offsets_kernel, dim3(1), dim3(64), 0, s, off, n);
  return hipGetLastError();
}

}  // namespace moe
