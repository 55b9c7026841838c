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

// Transposes into the weight gradients' operand layouts.  A block owns 64 destination
// columns q0 .. q0 + 63 of the padded layout: column q = poff[e] + i is row offsets[e] + i of
// the source while i < count_e, and zeros after.  Values pass through an LDS tile
// [64 columns][64 values] (bf16 pairs, padded rows): thread (j, part) = (tid / 4, tid % 4)
// puts values 16 part .. + 15 of column j, then takes value tid / 4 for columns
// 16 part .. + 15 and stores them as two 16-byte pieces:
//  plain : dst[c][q], row stride npad;
//  PACKED: matrix-core operand order (the weight-gradient GEMM's B operand), 1 KiB blocks
//          of 32 values of c x 16 columns q, ordered [c / 32][q / 16]; piece (c % 32) + 32 h
//          of a block holds columns 8 h .. + 7 of value c.
constexpr int kTransposeChunks = 4;
typedef uint32_t TileRow[33];

// Source row of each of the block's 64 columns (-1: padding), into srow.
__device__ __forceinline__ void tile_rows(const int32_t* __restrict__ row_map,
                                          const int32_t* __restrict__ offsets,
                                          const int32_t* __restrict__ poff, int E, int q0,
                                          int* srow) {
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
}

__device__ __forceinline__ void tile_put(TileRow* tile, int j, int part, const uint4& v0,
                                         const uint4& v1) {
  uint32_t* t = &tile[j][8 * part];
  t[0] = v0.x; t[1] = v0.y; t[2] = v0.z; t[3] = v0.w;
  t[4] = v1.x; t[5] = v1.y; t[6] = v1.z; t[7] = v1.w;
}

// Stores tile value cc (columns 16 part .. + 15) as destination value c.
template <bool PACKED>
__device__ __forceinline__ void tile_store(const TileRow* tile, int cc, int part, int c, int q0,
                                           int64_t npad, uint16_t* __restrict__ dst) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = tile[16 * part + 2 * i][cc >> 1], b = tile[16 * part + 2 * i + 1][cc >> 1];
    const int sh = 16 * (cc & 1);
    w[i] = ((a >> sh) & 0xFFFF) | (((b >> sh) & 0xFFFF) << 16);
  }
  if constexpr (PACKED) {
    uint4* blk = reinterpret_cast<uint4*>(dst) +
                 ((int64_t)(c >> 5) * (npad >> 4) + (q0 >> 4) + part) * 64;
    blk[c & 31] = make_uint4(w[0], w[1], w[2], w[3]);
    blk[(c & 31) + 32] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    uint4* d = reinterpret_cast<uint4*>(dst + (int64_t)c * npad + q0 + 16 * part);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// dst = src [rows, C] transposed into the padded layout (rows through row_map if given).
// A block takes up to kTransposeChunks chunks of 64 values of c: the source rows are found
// once and every chunk's loads (128 contiguous bytes of a source row each) are in flight
// together.
template <bool PACKED>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ src,
                                                            const int32_t* __restrict__ row_map,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ poff,
                                                            int E, int C, int64_t npad,
                                                            uint16_t* __restrict__ dst) {
  __shared__ TileRow tile[64];
  __shared__ int srow[64];
  const int q0 = blockIdx.x * 64, cb = blockIdx.y * 64 * kTransposeChunks;
  if (q0 >= poff[E]) return;  // block-uniform
  const int nch = min(kTransposeChunks, (C - cb) / 64);
  tile_rows(row_map, offsets, poff, E, q0, srow);
  __syncthreads();
  const int tid = threadIdx.x, j = tid >> 2, part = tid & 3;
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
    tile_put(tile, j, part, v[ch][0], v[ch][1]);
    __syncthreads();
    tile_store<PACKED>(tile, tid >> 2, part, cb + 64 * ch + (tid >> 2), q0, npad, dst);
  }
}

// SwiGLU backward on the interleaved gate|up rows (32-column blocks of g and u alternate),
// fused with the transposes its outputs need for the weight gradients.  Grid and column
// mapping as transpose_pad_kernel over the I values of a row, kSwigluChunks chunks of 64
// per block; per value, with s = sigma(g):
//   a = silu(g) u,  du = da silu(g),  dg = da u s (1 + g (1 - s))
// written as dgu (row-major, interleaved like gu: the data-gradient GEMM's input), dguT
// (packed, 2I values: the gate/up weight gradient's B operand) and aT (plain, I values: the
// down weight gradient's A operand); padding columns get zeros.
constexpr int kSwigluChunks = 2;
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t* __restrict__ gu,
                                                         const uint16_t* __restrict__ da,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ poff,
                                                         int E, int I, int64_t npad,
                                                         uint16_t* __restrict__ dgu,
                                                         uint16_t* __restrict__ dguT,
                                                         uint16_t* __restrict__ aT) {
  __shared__ TileRow tg[64], tu[64], ta[64];
  __shared__ int srow[64];
  const int q0 = blockIdx.x * 64, cb = blockIdx.y * 64 * kSwigluChunks;
  if (q0 >= poff[E]) return;  // block-uniform
  const int nch = min(kSwigluChunks, (I - cb) / 64);
  tile_rows(nullptr, offsets, poff, E, q0, srow);
  __syncthreads();
  const int tid = threadIdx.x, j = tid >> 2, part = tid & 3;
  const int r = srow[j];
  uint4 vg[kSwigluChunks][2], vu[kSwigluChunks][2], vd[kSwigluChunks][2];
#pragma unroll
  for (int ch = 0; ch < kSwigluChunks; ++ch) {
    vg[ch][0] = vg[ch][1] = vu[ch][0] = vu[ch][1] = vd[ch][0] = vd[ch][1] = make_uint4(0, 0, 0, 0);
    if (r >= 0 && ch < nch) {
      const int i0 = cb + 64 * ch + 16 * part;  // values i0 .. + 15, inside one 32-block
      const uint4* gp = reinterpret_cast<const uint4*>(gu + (int64_t)r * 2 * I + 64 * (i0 >> 5) +
                                                       (i0 & 31));
      const uint4* dp = reinterpret_cast<const uint4*>(da + (int64_t)r * I + i0);
      vg[ch][0] = gp[0];
      vg[ch][1] = gp[1];
      vu[ch][0] = gp[4];  // the up values sit 32 columns further
      vu[ch][1] = gp[5];
      vd[ch][0] = dp[0];
      vd[ch][1] = dp[1];
    }
  }
#pragma unroll
  for (int ch = 0; ch < kSwigluChunks; ++ch) {
    if (ch >= nch) break;  // block-uniform
    if (ch > 0) __syncthreads();  // the previous chunk's reads of the tiles are done
    uint4 og[2], ou[2], oa[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float g[8], u[8], d[8], fg[8], fu[8], fa[8];
      unpack8(vg[ch][h], g);
      unpack8(vu[ch][h], u);
      unpack8(vd[ch][h], d);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float s = 1.0f / (1.0f + __expf(-g[i]));
        const float silu = g[i] * s;
        fa[i] = silu * u[i];
        fu[i] = d[i] * silu;
        fg[i] = d[i] * u[i] * s * (1.0f + g[i] * (1.0f - s));
      }
      og[h] = pack8(fg);
      ou[h] = pack8(fu);
      oa[h] = pack8(fa);
    }
    if (r >= 0) {
      const int i0 = cb + 64 * ch + 16 * part;
      uint4* gp = reinterpret_cast<uint4*>(dgu + (int64_t)r * 2 * I + 64 * (i0 >> 5) + (i0 & 31));
      gp[0] = og[0];
      gp[1] = og[1];
      gp[4] = ou[0];
      gp[5] = ou[1];
    }
    tile_put(tg, j, part, og[0], og[1]);
    tile_put(tu, j, part, ou[0], ou[1]);
    tile_put(ta, j, part, oa[0], oa[1]);
    __syncthreads();
    const int cc = tid >> 2, i = cb + 64 * ch + cc;  // value i, columns 16 part .. + 15
    const int c = 64 * (i >> 5) + (i & 31);          // its gate column in the interleaved 2I
    tile_store<true>(tg, cc, part, c, q0, npad, dguT);
    tile_store<true>(tu, cc, part, c + 32, q0, npad, dguT);
    tile_store<false>(ta, cc, part, i, q0, npad, aT);
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
                             const int32_t* offsets, const int32_t* poff, int64_t npad, void* dgu,
                             void* dguT, void* aT, hipStream_t s) {
  const dim3 grid((unsigned)(npad / 64), (unsigned)div_up(p.I / 64, kSwigluChunks));
  hipLaunchKernelGGL(swiglu_bwd_kernel, grid, dim3(256), 0, s, (const uint16_t*)gu,
                     (const uint16_t*)da, offsets, poff, p.E, p.I, npad, (uint16_t*)dgu,
                     (uint16_t*)dguT, (uint16_t*)aT);
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
