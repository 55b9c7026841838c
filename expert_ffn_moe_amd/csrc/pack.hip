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

__global__ __launch_bounds__(256) void pack_bf16_kernel(const uint16_t* __restrict__ src0,
                                                        const uint16_t* __restrict__ src1,
                                                        int nmat, int E, int K, int N,
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
    const uint16_t* src = (m == 0) ? src0 : src1;
    const int col = nf * 32 + (L & 31);
    const int k0 = kf * 16 + 8 * (L >> 5);
    const uint16_t* p = src + (e * K + k0) * (size_t)N + col;
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = p[(size_t)i * N];
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
                     (const uint16_t*)wu, 2, p.E, p.H, p.I, (uint4*)packed_gu);
  hipLaunchKernelGGL(pack_bf16_kernel, grid, block, 0, s, (const uint16_t*)wd,
                     (const uint16_t*)nullptr, 1, p.E, p.I, p.H, (uint4*)packed_d);
  return hipGetLastError();
}

}  // namespace moe
