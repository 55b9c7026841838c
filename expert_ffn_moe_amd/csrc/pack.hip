// One-time weight packing for the matrix-core kernels.
//
// Natural layout: W_gate, W_up [E, H, I], W_down [E, I, H] (row-major, y = x W).  The
// packed layout stores, for every 32-column x 16-row (reduction) block of a matrix, one
// contiguous 1 KiB block in the order a 32x32x16 bf16 MFMA takes its B operand: lane L
// holds column L % 32, reduction rows 8 * (L / 32) .. + 8.  Blocks are ordered
//   gate/up: [e][n32][matrix: gate, up][k16][lane][8]   (n over I, k over H)
//   down   : [e][n32][k16][lane][8]                     (n over H, k over I)
// so a wavefront streaming one 32-column panel reads contiguous memory.
#include "moe_internal.h"

namespace moe {
namespace {

// Source of element (k, n) of matrix m of expert e, by layout:
//   kNatural : src_m[e][k][n]            ([E, K, N], the forward weights)
//   kTrans   : src0[e][n][k]             ([E, N, K]: the transpose of a forward matrix)
//   kGuTrans : the backward gate/up operand [E, K = 2I, N = H] whose reduction index k runs
//              over 32-column blocks of W_gate and W_up alternately (k = 64 b + j: j < 32 ->
//              W_gate[e][n][32 b + j], else W_up[e][n][32 b + j - 32]); src [E, H, I]
enum PackMode { kNatural = 0, kTrans = 1, kGuTrans = 2 };

__device__ __forceinline__ uint32_t pack_src(const uint16_t* src0, const uint16_t* src1, int mode,
                                             int m, size_t e, int K, int N, int k, int n) {
  if (mode == kNatural) return (m == 0 ? src0 : src1)[(e * K + k) * (size_t)N + n];
  if (mode == kTrans) return src0[(e * N + n) * (size_t)K + k];
  const int I = K / 2, b = k >> 6, j = k & 63;
  const uint16_t* s = j < 32 ? src0 : src1;
  return s[(e * N + n) * (size_t)I + 32 * b + (j & 31)];
}

__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint16_t* __restrict__ src0,
                                                        const uint16_t* __restrict__ src1,
                                                        int nmat, int E, int K, int N, int mode,
                                                        uint4* __restrict__ dst) {
  const int nk = K / 16, nn = N / 32;
  const size_t total = (size_t)E * nn * nmat * nk * 64;
  for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
       v += (size_t)gridDim.x * blockDim.x) {
    const int L = (int)(v % 64);
    size_t r = v / 64;
    const int kf = (int)(r % nk);
    r /= nk;
    const int m = (int)(r % nmat);
    r /= nmat;
    const int nf = (int)(r % nn);
    const size_t e = r / nn;
    const int col = nf * 32 + (L & 31);
    const int k0 = kf * 16 + 8 * (L >> 5);
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = pack_src(src0, src1, mode, m, e, K, N, k0 + i, col);
    uint4 o;
    o.x = h[0] | (h[1] << 16);
    o.y = h[2] | (h[3] << 16);
    o.z = h[4] | (h[5] << 16);
    o.w = h[6] | (h[7] << 16);
    dst[v] = o;
  }
}

}  // namespace

hipError_t launch_pack(const moe_problem& p, const void* wg, const void* wu, const void* wd,
                       void* packed_gu, void* packed_d, hipStream_t s) {
  if (p.w_dtype == MOE_F32) {
    const size_t n = (size_t)p.E * p.H * p.I * sizeof(float);
    hipError_t err = hipMemcpyAsync(packed_gu, wg, n, hipMemcpyDeviceToDevice, s);
    if (err == hipSuccess)
      err = hipMemcpyAsync((char*)packed_gu + n, wu, n, hipMemcpyDeviceToDevice, s);
    if (err == hipSuccess) err = hipMemcpyAsync(packed_d, wd, n, hipMemcpyDeviceToDevice, s);
    return err;
  }
  const dim3 grid(8192), block(256);
  hipLaunchKernelGGL(pack_bf16_kernel, grid, block, 0, s, (const uint16_t*)wg,
                     (const uint16_t*)wu, 2, p.E, p.H, p.I, (int)kNatural, (uint4*)packed_gu);
  hipLaunchKernelGGL(pack_bf16_kernel, grid, block, 0, s, (const uint16_t*)wd,
                     (const uint16_t*)nullptr, 1, p.E, p.I, p.H, (int)kNatural,
                     (uint4*)packed_d);
  return hipGetLastError();
}

// Backward operands: W_down^T as [E, K = H, N = I] (da = dyp W_down^T) and the interleaved
// [W_gate | W_up]^T as [E, K = 2I, N = H] (dxp = dgu [W_gate | W_up]^T).
hipError_t launch_pack_backward(const moe_problem& p, const void* wg, const void* wu,
                                const void* wd, void* packed_bwd_gu, void* packed_bwd_d,
                                hipStream_t s) {
  const dim3 grid(8192), block(256);
  hipLaunchKernelGGL(pack_bf16_kernel, grid, block, 0, s, (const uint16_t*)wd,
                     (const uint16_t*)nullptr, 1, p.E, p.H, p.I, (int)kTrans,
                     (uint4*)packed_bwd_d);
  hipLaunchKernelGGL(pack_bf16_kernel, grid, block, 0, s, (const uint16_t*)wg,
                     (const uint16_t*)wu, 1, p.E, 2 * p.I, p.H, (int)kGuTrans,
                     (uint4*)packed_bwd_gu);
  return hipGetLastError();
}

// A [E, K, N] matrix in its natural layout packed like the down weights (the router's
// W_r [E, H] as the operand [1, K = E, N = H] of dx += dlogits W_r).
hipError_t launch_pack_plain(int E, int K, int N, const void* w, void* packed, hipStream_t s) {
  hipLaunchKernelGGL(pack_bf16_kernel, dim3(8192), dim3(256), 0, s, (const uint16_t*)w,
                     (const uint16_t*)nullptr, 1, E, K, N, (int)kNatural, (uint4*)packed);
  return hipGetLastError();
}

}  // namespace moe
