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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// NT: the loads of yp and the stores of y carry the non-temporal hint (data used once).
template <bool NT>
__device__ __forceinline__ uint4 load_row(const uint4* p) {
  if constexpr (NT) {
    const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(q.x, q.y, q.z, q.w);
  }
  return *p;
}
template <bool NT>
__device__ __forceinline__ void store_row(uint4* p, const uint4& v) {
  if constexpr (NT)
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
  else
    *p = v;
}

// KMAX > 0: k <= KMAX, the k row loads of a vector are issued together before any of them
// is used (the slot loop unrolled); KMAX = 0: any k, one slot at a time.
template <int KMAX, bool NT>
__global__ __launch_bounds__(1024) void combine_bf16_kernel(const uint4* __restrict__ yp,
                                                           const float* __restrict__ w,
                                                           const int32_t* __restrict__ s2r,
                                                           int k, int nvec,
                                                           const uint4* __restrict__ shared,
                                                           uint4* __restrict__ y) {
  __shared__ int rows[32];
  __shared__ float wt[32];
  const int t = blockIdx.x;
  if ((int)threadIdx.x < k) {
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
        if (j < k && rows[j] >= 0) rv[j] = load_row<NT>(&yp[(size_t)rows[j] * nvec + v]);
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
        unpack8(load_row<NT>(&yp[(size_t)r * nvec + v]), f);
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
    store_row<NT>(&y[(size_t)t * nvec + v], pack8(acc));
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
  if ((int)threadIdx.x < k) {
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

template <int KMAX>
void combine_bf16(const moe_problem& p, const void* yp, const float* w, const int32_t* s2r,
                  const void* shared, void* y, hipStream_t s) {
  // One thread per 16-byte vector of a row when a row has at most 1024 of them (no idle
  // lanes in a last partial pass).  Past 256 MiB of yp (the size of the last-level cache)
  // the rows are streamed with the non-temporal hint: measured 429 -> 359 us on a
  // 131072 x 7168 yp, while on cache-sized yp the hint slowed the combine down.
  const int nvec = p.H / 8;
  const int threads = nvec <= 1024 ? (nvec + 63) / 64 * 64 : 256;
  const bool stream = (int64_t)p.T * p.k * p.H * 2 > ((int64_t)256 << 20);
  if (stream)
    hipLaunchKernelGGL((combine_bf16_kernel<KMAX, true>), dim3(p.T), dim3(threads), 0, s,
                       (const uint4*)yp, w, s2r, p.k, nvec, (const uint4*)shared, (uint4*)y);
  else
    hipLaunchKernelGGL((combine_bf16_kernel<KMAX, false>), dim3(p.T), dim3(threads), 0, s,
                       (const uint4*)yp, w, s2r, p.k, nvec, (const uint4*)shared, (uint4*)y);
}

}  // namespace

hipError_t launch_combine(const moe_problem& p, const void* yp, const float* w,
                          const int32_t* slot_to_row, const void* shared, void* y,
                          hipStream_t s) {
  if (p.act_dtype == MOE_F32)
    hipLaunchKernelGGL(combine_f32_kernel, dim3(p.T), dim3(256), 0, s, (const float4*)yp, w,
                       slot_to_row, p.k, p.H / 4, (const float4*)shared, (float4*)y);
  else if (p.k <= 4)
    combine_bf16<4>(p, yp, w, slot_to_row, shared, y, s);
  else if (p.k <= 8)
    combine_bf16<8>(p, yp, w, slot_to_row, shared, y, s);
  else
    combine_bf16<0>(p, yp, w, slot_to_row, shared, y, s);
  return hipGetLastError();
}

hipError_t launch_one_expert_offsets(int32_t* off, int n, hipStream_t s) {
  hipLaunchKernelGGL(one_expert_offsets_kernel, dim3(1), dim3(64), 0, s, off, n);
  return hipGetLastError();
}

}  // namespace moe
