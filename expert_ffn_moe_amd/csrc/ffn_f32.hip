// Grouped SwiGLU expert FFN in fp32 (vector ALU, fp32 fused multiply-add).  Used for the
// small fp32 problems; weights in the natural layout [E, H, I] / [E, I, H].
//   a[r]  = silu(xp[r] Wg[e]) * (xp[r] Wu[e]);  yp[r] = a[r] Wd[e]
// (with a row gather, x[row_token[r]] stands in for xp[r])
// One thread per output element; the row's expert is found by binary search over offsets.
#include "moe_internal.h"

namespace moe {
namespace {

// Largest e in [0, E) with offsets[e] <= r: the expert whose segment holds row r.
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int E, int r) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void gate_up_f32_kernel(const float* __restrict__ xp,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ offsets,
                                                          const float* __restrict__ wg,
                                                          const float* __restrict__ wu,
                                                          float* __restrict__ a, int E, int H,
                                                          int I) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int i = blockIdx.y * 64 + (threadIdx.x & 63);
  if (r >= offsets[E] || i >= I) return;
  const int e = expert_of_row(offsets, E, r);
  const float* x = xp + (size_t)(row_token ? row_token[r] : r) * H;
  const float* g = wg + (size_t)e * H * I + i;
  const float* u = wu + (size_t)e * H * I + i;
  float sg = 0.f, su = 0.f;
  for (int h = 0; h < H; ++h) {
    const float xv = x[h];
    sg = __builtin_fmaf(xv, g[(size_t)h * I], sg);
    su = __builtin_fmaf(xv, u[(size_t)h * I], su);
  }
  a[(size_t)r * I + i] = sg / (1.0f + expf(-sg)) * su;
}

__global__ __launch_bounds__(256) void down_f32_kernel(const float* __restrict__ a,
                                                       const int32_t* __restrict__ offsets,
                                                       const float* __restrict__ wd,
                                                       float* __restrict__ yp, int E, int H,
                                                       int I) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y * 64 + (threadIdx.x & 63);
  if (r >= offsets[E] || h >= H) return;
  const int e = expert_of_row(offsets, E, r);
  const float* av = a + (size_t)r * I;
  const float* w = wd + (size_t)e * I * H + h;
  float s = 0.f;
  for (int i = 0; i < I; ++i) s = __builtin_fmaf(av[i], w[(size_t)i * H], s);
  yp[(size_t)r * H + h] = s;
}

}  // namespace

hipError_t launch_gate_up_f32(const moe_problem& p, const float* xs, const int32_t* row_token,
                              const int32_t* offsets, const float* wg, const float* wu, float* a,
                              hipStream_t s) {
  const int rows = p.T * p.k;
  hipLaunchKernelGGL(gate_up_f32_kernel, dim3(div_up(rows, 4), div_up(p.I, 64)), dim3(256), 0,
                     s, xs, row_token, offsets, wg, wu, a, p.E, p.H, p.I);
  return hipGetLastError();
}

hipError_t launch_down_f32(const moe_problem& p, const float* a, const int32_t* offsets,
                           const float* wd, float* yp, hipStream_t s) {
  const int rows = p.T * p.k;
  hipLaunchKernelGGL(down_f32_kernel, dim3(div_up(rows, 4), div_up(p.H, 64)), dim3(256), 0, s,
                     a, offsets, wd, yp, p.E, p.H, p.I);
  return hipGetLastError();
}

}  // namespace moe
