// Backward pass of the layer (docs.axolotl.ai "integrations.expert_parallel.args", attribute
// table, row `expert_parallel_save_dispatch`: the backward reuses the forward's saved
// routing -- top-k and the split counts -- and the dispatch rows, saved or recomputed).
//
// With r = slot_to_row[t, j] for the kept slots, g|u = x[t] [W_gate | W_up], a = silu(g) u,
// yp = a W_down:
//   combine backward   dyp[r] = w[t,j] dy[t]             dw[t,j] = <yp[r], dy[t]>
//   down backward      da = dyp W_down^T                  dW_down[e] = a_e^T dyp_e
//   SwiGLU backward    du = da silu(g)                    dg = da u sigma(g) (1 + g (1 - sigma(g)))
//   gate/up backward   dxp = [dg | du] [W_gate | W_up]^T  dW_gate|up[e] = x_e^T [dg | du]_e
//   dispatch backward  dx[t] = sum over kept slots of dxp[r]
// The data-gradient GEMMs run on the forward's grouped-GEMM kernels with operands packed for
// the backward (W_down^T, the interleaved [W_gate | W_up]^T).  The weight gradients reduce
// over each expert's rows: the row-major [rows, C] operands are transposed into [C, rows]
// with every expert's rows padded to a multiple of 16 (zeros), so that the reduction
// dimension is contiguous for both matrix-core operands, and a grouped GEMM per expert
// accumulates in fp32.
#include <algorithm>

#include "bf16.h"
#include "moe_internal.h"
#include "wave.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// One token per block: dyp rows of its kept slots and the gradient of its routing weights.
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint4* __restrict__ dy,
                                                          const uint4* __restrict__ yp,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ s2r,
                                                          int k, int nvec,
                                                          uint4* __restrict__ dyp,
                                                          float* __restrict__ dw) {
  __shared__ int rows[32];
  __shared__ float wt[32];
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < k) {
    rows[tid] = s2r[(size_t)t * k + tid];
    wt[tid] = w[(size_t)t * k + tid];
  }
  float f[4][8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int v = tid + 256 * q;
    if (v < nvec) unpack8(dy[(size_t)t * nvec + v], f[q]);
  }
  __syncthreads();
  for (int j = 0; j < k; ++j) {
    const int r = rows[j];  // block-uniform
    if (r < 0) {
      if (tid == 0) dw[(size_t)t * k + j] = 0.0f;
      continue;
    }
    const float wj = wt[j];
    float dot = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int v = tid + 256 * q;
      if (v < nvec) {
        float y8[8], o[8];
        unpack8(yp[(size_t)r * nvec + v], y8);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          o[i] = wj * f[q][i];
          dot = __builtin_fmaf(y8[i], f[q][i], dot);
        }
        dyp[(size_t)r * nvec + v] = pack8(o);
      }
    }
    dot = wave_sum(dot);
    if ((tid & 63) == 0) red[tid >> 6] = dot;
    __syncthreads();
    if (tid == 0) dw[(size_t)t * k + j] = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
  }
}

// SwiGLU backward on the interleaved gate|up rows (32-column blocks of g and u alternate),
// for the layout's rows r < offsets[E]: dgu (same interleaving) and the recomputed a.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint4* __restrict__ gu,
                                                         const uint4* __restrict__ da,
                                                         const int32_t* __restrict__ nrows,
                                                         int I, uint4* __restrict__ dgu,
                                                         uint4* __restrict__ a) {
  const int per_row = I / 8;
  const int64_t total = (int64_t)(*nrows) * per_row;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = q / per_row;
    const int c8 = (int)(q - r * per_row);
    const int i0 = 8 * c8, b = i0 >> 5, j0 = i0 & 31;
    const int64_t gv = (r * 2 * I + 64 * b + j0) / 8;  // uint4 index of g; u is 4 further
    float g[8], u[8], d[8], og[8], ou[8], oa[8];
    unpack8(gu[gv], g);
    unpack8(gu[gv + 4], u);
    unpack8(da[r * per_row + c8], d);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float s = 1.0f / (1.0f + __expf(-g[i]));
      const float silu = g[i] * s;
      oa[i] = silu * u[i];
      ou[i] = d[i] * silu;
      og[i] = d[i] * u[i] * s * (1.0f + g[i] * (1.0f - s));
    }
    dgu[gv] = pack8(og);
    dgu[gv + 4] = pack8(ou);
    a[r * per_row + c8] = pack8(oa);
  }
}

// poff[e] = sum over e' < e of roundup16(offsets[e' + 1] - offsets[e']), poff[E] the total
// (E <= 1024, one block).
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int32_t* __restrict__ poff) {
  __shared__ int s[1024];
  const int e = threadIdx.x;
  const int c = e < E ? ((offsets[e + 1] - offsets[e] + 15) & ~15) : 0;
  s[e] = c;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = e >= d ? s[e - d] : 0;
    __syncthreads();
    s[e] += v;
    __syncthreads();
  }
  if (e < E) poff[e] = s[e] - c;
  if (e == E - 1) poff[E] = s[e];
}

// dst[c][poff[e] + r - offsets[e]] = src[row r][c] (src row = row_map[r] if row_map), for
// the layout rows r < offsets[E]; 64 rows x 64 columns per block through LDS.
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ src,
                                                            const int32_t* __restrict__ row_map,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ poff,
                                                            int E, int C, int64_t npad,
                                                            uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[64][64 + 8];
  __shared__ int prow[64];
  const int n = offsets[E];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  if (r0 >= n) return;  // block-uniform
  const int tid = threadIdx.x;
  {
    const int rr = tid >> 2, part = tid & 3;
    const int r = r0 + rr;
    if (r < n) {
      const int64_t sr = row_map ? row_map[r] : r;
      const uint4* p = reinterpret_cast<const uint4*>(src + sr * C + c0 + 16 * part);
      const uint4 v0 = p[0], v1 = p[1];
      uint32_t wv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        tile[rr][16 * part + 2 * i] = (uint16_t)(wv[i] & 0xFFFF);
        tile[rr][16 * part + 2 * i + 1] = (uint16_t)(wv[i] >> 16);
      }
      if (part == 0) {
        int lo = 0, hi = E;  // expert of row r: the largest e with offsets[e] <= r
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (offsets[mid] <= r) lo = mid; else hi = mid;
        }
        prow[rr] = poff[lo] + r - offsets[lo];
      }
    }
  }
  __syncthreads();
  const int cc = tid >> 2, part = tid & 3;
  uint16_t* d = dst + (int64_t)(c0 + cc) * npad;
#pragma unroll 4
  for (int i = 0; i < 16; ++i) {
    const int rr = 16 * part + i;
    if (r0 + rr < n) d[prow[rr]] = tile[rr][cc];
  }
}

// Zeros in the padding columns [poff[e] + count_e, poff[e + 1]) of every row c < C.
__global__ __launch_bounds__(256) void zero_pad_kernel(const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ poff, int C,
                                                       int64_t npad, uint16_t* __restrict__ dst) {
  const int e = blockIdx.x;
  const int c0 = poff[e] + offsets[e + 1] - offsets[e], c1 = poff[e + 1];
  const int w = c1 - c0;  // < 16
  if (w <= 0) return;
  for (int q = threadIdx.x; q < C * w; q += blockDim.x) {
    const int c = q / w;
    dst[(int64_t)c * npad + c0 + (q - c * w)] = 0;
  }
}

// Weight gradient of every expert: out[e][m][n] = sum over its (padded) rows k of
// AT[m][k] BT[n][k], fp32 (rows m >= M of the last tile are computed on clamped operands
// and not stored).  A block of 4 wavefronts takes a 128 x 128 tile of one expert,
// each wavefront 64 x 64 (2 x 2 accumulators of 32x32x16 bf16 MFMAs), operands loaded
// straight from memory (both have the reduction dimension contiguous).  gu_split: the n
// dimension is the interleaved gate|up one (2I): columns go to out (gate) or out2 (up),
// each [E][M][I].
__global__ __launch_bounds__(256) void wgrad_kernel(const uint16_t* __restrict__ AT,
                                                    const uint16_t* __restrict__ BT,
                                                    const int32_t* __restrict__ poff, int M,
                                                    int Ncols, int64_t npad, int gu_split,
                                                    float* __restrict__ out,
                                                    float* __restrict__ out2) {
  const int e = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int mb = blockIdx.x * 128 + (wave & 1) * 64;
  const int nb = blockIdx.y * 128 + (wave >> 1) * 64;
  const int k0 = poff[e], k1 = poff[e + 1];
  const uint16_t* ap[2];
  const uint16_t* bp[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    ap[i] = AT + (int64_t)min(mb + 32 * i + (lane & 31), M - 1) * npad + 8 * (lane >> 5);
    bp[i] = BT + (int64_t)(nb + 32 * i + (lane & 31)) * npad + 8 * (lane >> 5);
  }
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16_t{};
  if (k1 > k0) {
    uint4 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = *(const uint4*)(ap[i] + k0);
      b[i] = *(const uint4*)(bp[i] + k0);
    }
    for (int k = k0; k < k1; k += 16) {
      const int kn = min(k + 16, k1 - 16);  // the last step reloads its own operands
      uint4 an[2], bn[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        an[i] = *(const uint4*)(ap[i] + kn);
        bn[i] = *(const uint4*)(bp[i] + kn);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, a[i]), __builtin_bit_cast(bf16x8_t, b[j]), acc[i][j],
              0, 0, 0);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = an[i];
        b[i] = bn[i];
      }
    }
  }
  // accumulator element q of lane l: row 8 (q / 4) + 4 (l / 32) + q % 4, column l % 32
  const int I = Ncols / 2;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = mb + 32 * i + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
        const int n = nb + 32 * j + (lane & 31);
        if (m >= M) continue;
        if (!gu_split) {
          out[((int64_t)e * M + m) * Ncols + n] = acc[i][j][q];
        } else {
          const int blk = n >> 6, jj = n & 63;
          float* o = jj < 32 ? out : out2;
          o[((int64_t)e * M + m) * I + 32 * blk + (jj & 31)] = acc[i][j][q];
        }
      }
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ in,
                                                          int64_t n, uint16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = to_bf16(in[i]);
}

int grid_for(int64_t work, int per_block) {
  return (int)std::max<int64_t>(1, std::min<int64_t>(div_up64(work, per_block), 8192));
}

}  // namespace

hipError_t launch_combine_bwd(const moe_problem& p, const void* dy, const void* yp,
                              const float* w, const int32_t* slot_to_row, void* dyp, float* dw,
                              hipStream_t s) {
  hipLaunchKernelGGL(combine_bwd_kernel, dim3(p.T), dim3(256), 0, s, (const uint4*)dy,
                     (const uint4*)yp, w, slot_to_row, p.k, p.H / 8, (uint4*)dyp, dw);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const moe_problem& p, const void* gu, const void* da,
                             const int32_t* offsets, void* dgu, void* a, hipStream_t s) {
  const int64_t work = (int64_t)p.T * p.k * (p.I / 8);
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(grid_for(work, 256)), dim3(256), 0, s,
                     (const uint4*)gu, (const uint4*)da, offsets + p.E, p.I, (uint4*)dgu,
                     (uint4*)a);
  return hipGetLastError();
}

hipError_t launch_pad_offsets(const int32_t* offsets, int E, int32_t* poff, hipStream_t s) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(1024), 0, s, offsets, E, poff);
  return hipGetLastError();
}

hipError_t launch_transpose_pad(const void* src, const int32_t* row_map, const int32_t* offsets,
                                const int32_t* poff, int E, int64_t max_rows, int C,
                                int64_t npad, void* dst, hipStream_t s) {
  const dim3 grid((unsigned)div_up64(max_rows, 64), (unsigned)(C / 64));
  hipLaunchKernelGGL(transpose_pad_kernel, grid, dim3(256), 0, s, (const uint16_t*)src, row_map,
                     offsets, poff, E, C, npad, (uint16_t*)dst);
  hipLaunchKernelGGL(zero_pad_kernel, dim3(E), dim3(256), 0, s, offsets, poff, C, npad,
                     (uint16_t*)dst);
  return hipGetLastError();
}

hipError_t launch_wgrad(const void* AT, const void* BT, const int32_t* poff, int E, int M,
                        int Ncols, int64_t npad, bool gu_split, float* out, float* out2,
                        hipStream_t s) {
  const dim3 grid(div_up(M, 128), Ncols / 128, E);
  hipLaunchKernelGGL(wgrad_kernel, grid, dim3(256), 0, s, (const uint16_t*)AT,
                     (const uint16_t*)BT, poff, M, Ncols, npad, gu_split ? 1 : 0, out, out2);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* in, int64_t n, void* out, hipStream_t s) {
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, in, n,
                     (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace moe
