// FP8 quantisation: OCP E4M3 codes with UE8M0 (power-of-two) scales, one scale per block
// of 32 consecutive elements along a GEMM's reduction dimension.
//
// LightLLM PR #1687 (PR body and the walkthrough's grouped-MoE row): the grouped GEMMs take
// FP8 operands with UE8M0 scales, and the SwiGLU output is quantised on the prefix-sum
// layout before the down projection.  The pages leave the block size open; 32 along the
// reduction dimension is the block of the gfx950 scaled matrix-core instruction.
//
// A block with absolute maximum amax gets the scale 2^e, e the smallest integer with
// amax <= 448 * 2^e (so nothing saturates; 0 for an all-zero block), stored as the byte
// e + 127; each element is rounded to the nearest E4M3 value of element * 2^-e, ties to
// even (the hardware conversion).
#include <algorithm>

#include "bf16.h"
#include "fp8.h"
#include "moe_internal.h"

namespace moe {
namespace {

// Rows of bf16 [rows, 32 * kb] -> codes [rows, 32 * kb], scales [rows, kb]; one thread per
// block of 32 (64 contiguous input bytes).  With row_limit, rows >= *row_limit (read on
// the device) are skipped.
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ in,
                                                         int64_t nblocks, int kb,
                                                         const int32_t* __restrict__ row_limit,
                                                         uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
  if (row_limit) nblocks = min(nblocks, (int64_t)max(*row_limit, 0) * kb);
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblocks;
       b += (int64_t)gridDim.x * blockDim.x) {
    const uint4* src = reinterpret_cast<const uint4*>(in + b * kQBlock);
    float f[kQBlock];
#pragma unroll
    for (int q = 0; q < 4; ++q) unpack8(src[q], f + 8 * q);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kQBlock; ++i) amax = fmaxf(amax, fabsf(f[i]));
    const int e = ue8m0_exp(amax);
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = pack_fp8x4(f + 4 * q, -e);
    uint4* dst = reinterpret_cast<uint4*>(codes + b * kQBlock);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    scales[b] = (uint8_t)(e + 127);
  }
}

// Weights bf16 [E, K, N] (K the reduction dimension) -> matrix-core operand blocks of the
// 32x32x64 scaled FP8 instruction: per (expert, 32-column panel n32, matrix m, k-step of
// 64) 2 KiB in which lane L (column L % 32, half h = L / 32) holds 32 bytes: k = 16h .. +16
// then k = 32 + 16h .. +16 of the k-step.  Lane L supplies the scale of its column's
// 32-element block h of the k-step; scale bytes are grouped per lane by 4 k-steps.
//   codes : [E][N/32][nmat][K/64][64 lanes][32 B]
//   scales: [E][N/32][nmat][ceil(K/256)][64 lanes][4 B]
__global__ __launch_bounds__(256) void pack_fp8_kernel(const uint16_t* __restrict__ src0,
                                                       const uint16_t* __restrict__ src1,
                                                       int nmat, int E, int K, int N,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales) {
  const int nks = K / 64, nkg = div_up(nks, 4), nn = N / 32;
  const int64_t total = (int64_t)E * nn * nmat * nks * 64;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int L = (int)(v % 64);
    int64_t r = v / 64;
    const int ks = (int)(r % nks);
    r /= nks;
    const int m = (int)(r % nmat);
    r /= nmat;
    const int nf = (int)(r % nn);
    const int64_t e = r / nn;
    const uint16_t* src = (m == 0) ? src0 : src1;
    const int col = nf * 32 + (L & 31), h = L >> 5;
    const uint16_t* p = src + (e * K + (int64_t)ks * 64) * N + col;
    float blk[2][kQBlock];
    float amax[2] = {0.0f, 0.0f};
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < kQBlock; ++i) {
        blk[b][i] = bf16_lo((uint32_t)p[(int64_t)(32 * b + i) * N]);
        amax[b] = fmaxf(amax[b], fabsf(blk[b][i]));
      }
    const int e0 = ue8m0_exp(amax[0]), e1 = ue8m0_exp(amax[1]);
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = pack_fp8x4(&blk[0][16 * h + 4 * q], -e0);
#pragma unroll
    for (int q = 0; q < 4; ++q) w[4 + q] = pack_fp8x4(&blk[1][16 * h + 4 * q], -e1);
    uint4* dst = reinterpret_cast<uint4*>(codes + v * 32);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    const int64_t panel = (e * nn + nf) * nmat + m;
    uint8_t* sc = scales + ((panel * nkg + ks / 4) * 64 + L) * 4;
    sc[ks % 4] = (uint8_t)((h ? e1 : e0) + 127);
    if (ks == nks - 1)  // unused bytes of the last group
      for (int j = ks % 4 + 1; j < 4; ++j) sc[j] = 127;
  }
}

}  // namespace

size_t fp8_packed_code_bytes(int E, int K, int N, int nmat) {
  return (size_t)E * (N / 32) * nmat * (K / 64) * 2048;
}
size_t fp8_packed_scale_bytes(int E, int K, int N, int nmat) {
  return (size_t)E * (N / 32) * nmat * div_up(K / 64, 4) * 256;
}

hipError_t launch_pack_fp8(const moe_problem& p, const void* wg, const void* wu, const void* wd,
                           void* packed_gu, void* packed_d, hipStream_t s) {
  uint8_t* gu = (uint8_t*)packed_gu;
  uint8_t* d = (uint8_t*)packed_d;
  const dim3 grid(8192), block(256);
  hipLaunchKernelGGL(pack_fp8_kernel, grid, block, 0, s, (const uint16_t*)wg, (const uint16_t*)wu,
                     2, p.E, p.H, p.I, gu, gu + align256(fp8_packed_code_bytes(p.E, p.H, p.I, 2)));
  hipLaunchKernelGGL(pack_fp8_kernel, grid, block, 0, s, (const uint16_t*)wd,
                     (const uint16_t*)nullptr, 1, p.E, p.I, p.H, d,
                     d + align256(fp8_packed_code_bytes(p.E, p.I, p.H, 1)));
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* in, int64_t rows, int K, const int32_t* row_limit,
                             uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nblocks = rows * (K / kQBlock);
  if (nblocks == 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>(div_up64(nblocks, 256), 4096);
  hipLaunchKernelGGL(quant_rows_kernel, dim3(grid), dim3(256), 0, s, (const uint16_t*)in,
                     nblocks, K / kQBlock, row_limit, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
