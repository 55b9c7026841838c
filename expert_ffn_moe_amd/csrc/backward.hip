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
// with every expert's rows padded to a multiple of 64 (zeros), so that the reduction
// dimension is contiguous for both matrix-core operands, and the prefill GEMM tile
// (launch_wgrad_bf16) accumulates each expert's gradient in fp32.
#include <algorithm>

#include "bf16.h"
#include "moe_internal.h"
#include "wave.h"

namespace moe {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// One token per block: dyp rows of its kept slots and the gradient of its routing weights.
// The slots are independent (no barrier between them, so the loads of several slots can be
// in flight together); each wavefront leaves its partial dot product per slot in LDS and one
// barrier at the end precedes the per-slot sums.
__global__ __launch_bounds__(256) void combine_bwd_kernel(const uint4* __restrict__ dy,
                                                          const uint4* __restrict__ yp,
                                                          const float* __restrict__ w,
                                                          const int32_t* __restrict__ s2r,
                                                          int k, int nvec,
                                                          uint4* __restrict__ dyp,
                                                          float* __restrict__ dw) {
  __shared__ float red[32][4];
  const int t = blockIdx.x, tid = threadIdx.x;
  float f[4][8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int v = tid + 256 * q;
    if (v < nvec) unpack8(dy[(size_t)t * nvec + v], f[q]);
  }
#pragma unroll 4
  for (int j = 0; j < k; ++j) {
    const int r = s2r[(size_t)t * k + j];  // block-uniform
    const float wj = w[(size_t)t * k + j];
    float dot = 0.0f;
    if (r >= 0) {
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
    }
    dot = wave_sum(dot);
    if ((tid & 63) == 0) red[j][tid >> 6] = dot;
  }
  __syncthreads();
  if (tid < k)
    dw[(size_t)t * k + tid] = s2r[(size_t)t * k + tid] < 0
                                  ? 0.0f
                                  : (red[tid][0] + red[tid][1]) + (red[tid][2] + red[tid][3]);
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

// poff[e] = sum over e' < e of the count of e' rounded up to a multiple of gran, poff[E]
// the total (E <= 1024, one block).
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int gran,
                                                           int32_t* __restrict__ poff) {
  __shared__ int s[1024];
  const int e = threadIdx.x;
  const int c = e < E ? (offsets[e + 1] - offsets[e] + gran - 1) / gran * gran : 0;
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

// dst[c][q] for the padded columns q of a block: column q = poff[e] + i holds src row
// offsets[e] + i (through row_map if given) while i < count_e, zeros after.  A block takes
// 64 destination columns x up to kTransposeChunks chunks of 64 values of c: it finds the
// source rows once, loads every chunk (128 contiguous bytes of each source row per chunk,
// all in flight together), then per chunk stores 64 destination rows (128 contiguous bytes
// each) through LDS.
// PACKED: dst in matrix-core operand order instead (the weight-gradient GEMM's B operand):
// 1 KiB blocks of 32 values of c x 16 columns q, ordered [c / 32][q / 16]; piece
// (c % 32) + 32 h of a block holds columns 8 h .. + 7 of value c.
constexpr int kTransposeChunks = 4;

template <bool PACKED>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ src,
                                                            const int32_t* __restrict__ row_map,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ poff,
                                                            int E, int C, int64_t npad,
                                                            uint16_t* __restrict__ dst) {
  __shared__ uint32_t tile[64][33];  // [destination column][pairs of c], padded row
  __shared__ int srow[64];
  const int q0 = blockIdx.x * 64, cb = blockIdx.y * 64 * kTransposeChunks;
  const int nch = min(kTransposeChunks, (C - cb) / 64);
  if (q0 >= poff[E]) return;  // block-uniform
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int q = q0 + tid;
    int lo = 0, hi = E;  // expert of column q: the largest e with poff[e] <= q
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (poff[mid] <= q) lo = mid; else hi = mid;
    }
    const int r = offsets[lo] + (q - poff[lo]);
    srow[tid] = r < offsets[lo + 1] ? (row_map ? row_map[r] : r) : -1;
  }
  __syncthreads();
  const int j = tid >> 2, part = tid & 3;  // load: column j, values 16 part .. + 15 of a chunk
  uint4 v[kTransposeChunks][2];
  {
    const int r = srow[j];
#pragma unroll
    for (int ch = 0; ch < kTransposeChunks; ++ch) {
      v[ch][0] = v[ch][1] = make_uint4(0, 0, 0, 0);
      if (r >= 0 && ch < nch) {
        const uint4* p =
            reinterpret_cast<const uint4*>(src + (int64_t)r * C + cb + 64 * ch + 16 * part);
        v[ch][0] = p[0];
        v[ch][1] = p[1];
      }
    }
  }
#pragma unroll
  for (int ch = 0; ch < kTransposeChunks; ++ch) {
    if (ch >= nch) break;  // block-uniform
    if (ch > 0) __syncthreads();  // the previous chunk's reads of the tile are done
    {
      uint32_t* t = &tile[j][8 * part];
      t[0] = v[ch][0].x; t[1] = v[ch][0].y; t[2] = v[ch][0].z; t[3] = v[ch][0].w;
      t[4] = v[ch][1].x; t[5] = v[ch][1].y; t[6] = v[ch][1].z; t[7] = v[ch][1].w;
    }
    __syncthreads();
    const int c0 = cb + 64 * ch;
    const int cc = tid >> 2;  // store: value c0 + cc, columns 16 part .. + 15
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = tile[16 * part + 2 * i][cc >> 1], b = tile[16 * part + 2 * i + 1][cc >> 1];
      const int sh = 16 * (cc & 1);
      w[i] = ((a >> sh) & 0xFFFF) | (((b >> sh) & 0xFFFF) << 16);
    }
    if constexpr (PACKED) {
      const int c = c0 + cc;
      uint4* blk = reinterpret_cast<uint4*>(dst) +
                   ((int64_t)(c >> 5) * (npad >> 4) + (q0 >> 4) + part) * 64;
      blk[c & 31] = make_uint4(w[0], w[1], w[2], w[3]);
      blk[(c & 31) + 32] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      uint4* d = reinterpret_cast<uint4*>(dst + (int64_t)(c0 + cc) * npad + q0 + 16 * part);
      d[0] = make_uint4(w[0], w[1], w[2], w[3]);
      d[1] = make_uint4(w[4], w[5], w[6], w[7]);
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

hipError_t launch_pad_offsets(const int32_t* offsets, int E, int gran, int32_t* poff,
                              hipStream_t s) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(1024), 0, s, offsets, E, gran, poff);
  return hipGetLastError();
}

hipError_t launch_transpose_pad(const void* src, const int32_t* row_map, const int32_t* offsets,
                                const int32_t* poff, int E, int C, int64_t npad, bool packed,
                                void* dst, hipStream_t s) {
  const dim3 grid((unsigned)(npad / 64), (unsigned)div_up(C / 64, kTransposeChunks));
  if (packed)
    hipLaunchKernelGGL(transpose_pad_kernel<true>, grid, dim3(256), 0, s, (const uint16_t*)src,
                       row_map, offsets, poff, E, C, npad, (uint16_t*)dst);
  else
    hipLaunchKernelGGL(transpose_pad_kernel<false>, grid, dim3(256), 0, s, (const uint16_t*)src,
                       row_map, offsets, poff, E, C, npad, (uint16_t*)dst);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* in, int64_t n, void* out, hipStream_t s) {
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, in, n,
                     (uint16_t*)out);
  return hipGetLastError();
}

}  // namespace moe
