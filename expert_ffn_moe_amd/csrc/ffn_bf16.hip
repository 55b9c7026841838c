// Grouped SwiGLU expert FFN in bf16 on the gfx950 matrix cores (fp32 accumulation).
//
// LightLLM PR #1687 (PR body): the expert GEMMs run on the expert prefix-sum layout,
// followed by `silu_and_mul`; the row count of every expert is data dependent and is
// read on the device from `offsets`.
//
//   gate/up: a[r]  = silu(xp[r] Wg[e]) * (xp[r] Wu[e])     (SwiGLU fused in the epilogue)
//   down   : yp[r] = a[r] Wd[e]
//
// Two kernel shapes, chosen from the problem shape:
//  * prefill (many rows per expert): 128-row M tiles listed in a device-built tile table;
//    the activation tile goes through LDS (shared by the 8 wavefronts of the block) and
//    each wavefront streams its own weight panels straight from HBM into registers in
//    matrix-core operand order (the packed layout makes each operand a contiguous 1 KiB).
//    v_mfma_f32_32x32x16_bf16.
//  * decode (a few rows per expert): a weight-streaming kernel; one wavefront per
//    32/64-column panel of one expert, 16-row M steps, v_mfma_f32_16x16x32_bf16.
#include "bf16.h"
#include "moe_internal.h"
#include "wave.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

constexpr int kOperandElems = 512;  // one packed 32x16 (or 16x32) operand block

// ------------------------------------------------------------------------------------
// Tile table: expert e with c rows gets ceil(c / 128) consecutive tiles.
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ offsets,
                                                          int E, int32_t* __restrict__ count,
                                                          int32_t* __restrict__ tile_expert,
                                                          int32_t* __restrict__ tile_row0) {
  __shared__ int wsum[16];
  const int e = threadIdx.x, wave = e >> 6, lane = e & 63;
  int n = 0, o = 0;
  if (e < E) {
    o = offsets[e];
    n = div_up(offsets[e + 1] - o, kPrefillBM);
  }
  const int inc = wave_inclusive_scan(n);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  const int start = base + inc - n;
  for (int m = 0; m < n; ++m) {
    tile_expert[start + m] = e;
    tile_row0[start + m] = o + m * kPrefillBM;
  }
  if (e == E - 1) count[0] = base + inc;
}

// ------------------------------------------------------------------------------------
// Prefill grouped GEMM.  Block = 8 wavefronts, tile = 128 rows x 8 panels.
//   GATE_UP: panel = 32 output columns of `a` = one gate and one up operand column.
//   DOWN   : panel = 64 output columns of yp = two operand columns.
// K steps of 64 (4 MFMA k-steps); LDS double-buffers the activation tile.
// ------------------------------------------------------------------------------------
template <bool GATE_UP>
__global__ __launch_bounds__(512) void prefill_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_count, const int32_t* __restrict__ tile_expert,
    const int32_t* __restrict__ tile_row0, const uint16_t* __restrict__ Bp,
    uint16_t* __restrict__ out, int K, int Nout, int ntn) {
  __shared__ uint4 lds_a[2][16 * 64];  // [buf][(m32 * 4 + k16) * 64 + lane]

  // linear block index -> (M tile, N panel group), N fastest so that the blocks sharing
  // an activation tile run together
  const int mt = blockIdx.x / ntn;
  const int nt = blockIdx.x - mt * ntn;
  if (mt >= tile_count[0]) return;  // block-uniform
  const int e = tile_expert[mt];
  const int row0 = tile_row0[mt];
  const int rows = min(kPrefillBM, offsets[e + 1] - row0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nk16 = K / 16;
  const int nf32 = Nout / 32;

  // this wavefront's two operand columns (clamped when the panel lies past Nout)
  int col0;
  bool active;
  const uint16_t* b0;
  const uint16_t* b1;
  if (GATE_UP) {
    int af = nt * 8 + wave;
    active = af < nf32;
    af = min(af, nf32 - 1);
    col0 = af * 32;
    b0 = Bp + (size_t)(e * nf32 + af) * 2 * nk16 * kOperandElems;
    b1 = b0 + (size_t)nk16 * kOperandElems;
  } else {
    int nf = nt * 16 + 2 * wave;
    active = nf < nf32;
    nf = min(nf, nf32 - 2);
    col0 = nf * 32;
    b0 = Bp + (size_t)(e * nf32 + nf) * nk16 * kOperandElems;
    b1 = b0 + (size_t)nk16 * kOperandElems;
  }
  b0 += lane * 8;
  b1 += lane * 8;

  // activation tile loader: 1024 16-byte pieces, two per thread
  const uint16_t* ag[2];
  int lds_slot[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int idx = threadIdx.x + 512 * p;
    const int r = idx >> 3, q = idx & 7;
    ag[p] = A + (size_t)(row0 + min(r, rows - 1)) * K + q * 8;
    lds_slot[p] = ((r >> 5) * 4 + (q >> 1)) * 64 + (r & 31) + 32 * (q & 1);
  }

  f32x16_t acc0[4], acc1[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    acc0[m] = f32x16_t{};
    acc1[m] = f32x16_t{};
  }

  const int nkt = K / 64;
  uint4 areg[2], bcur[4][2], bnext[4][2];
#pragma unroll
  for (int p = 0; p < 2; ++p) areg[p] = *(const uint4*)(ag[p]);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bcur[kk][0] = *(const uint4*)(b0 + (size_t)kk * kOperandElems);
    bcur[kk][1] = *(const uint4*)(b1 + (size_t)kk * kOperandElems);
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) lds_a[0][lds_slot[p]] = areg[p];
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) {
#pragma unroll
      for (int p = 0; p < 2; ++p) areg[p] = *(const uint4*)(ag[p] + (size_t)(kt + 1) * 64);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const size_t o = (size_t)((kt + 1) * 4 + kk) * kOperandElems;
        bnext[kk][0] = *(const uint4*)(b0 + o);
        bnext[kk][1] = *(const uint4*)(b1 + o);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_t a[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) a[m] = as_bf16x8(lds_a[cur][(m * 4 + kk) * 64 + lane]);
      const bf16x8_t bb0 = as_bf16x8(bcur[kk][0]);
      const bf16x8_t bb1 = as_bf16x8(bcur[kk][1]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc0[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], bb0, acc0[m], 0, 0, 0);
        acc1[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], bb1, acc1[m], 0, 0, 0);
      }
    }
    if (more) {
#pragma unroll
      for (int p = 0; p < 2; ++p) lds_a[cur ^ 1][lds_slot[p]] = areg[p];
    }
    __syncthreads();
    if (more) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        bcur[kk][0] = bnext[kk][0];
        bcur[kk][1] = bnext[kk][1];
      }
    }
  }

  if (!active) return;
  // 32x32 accumulator layout: element i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32.
  const int c = col0 + (lane & 31);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = m * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      if (r < rows) {
        uint16_t* o = out + (size_t)(row0 + r) * Nout;
        if (GATE_UP) {
          o[c] = to_bf16(silu_mul(acc0[m][i], acc1[m][i]));
        } else {
          o[c] = to_bf16(acc0[m][i]);
          o[c + 32] = to_bf16(acc1[m][i]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// Decode (weight streaming).  One wavefront per panel of one expert:
//   GATE_UP: 32 columns of `a` (gate + up operand columns); DOWN: 64 columns of yp.
// Each k-step of 32 issues 4 B operand loads (16 columns each) and one A load.
// ------------------------------------------------------------------------------------
template <bool GATE_UP>
__global__ __launch_bounds__(256) void decode_kernel(const uint16_t* __restrict__ A,
                                                     const int32_t* __restrict__ offsets,
                                                     const uint16_t* __restrict__ Bp,
                                                     uint16_t* __restrict__ out, int K,
                                                     int Nout) {
  const int e = blockIdx.y;
  const int row_beg = offsets[e];
  const int cnt = offsets[e + 1] - row_beg;
  if (cnt <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + wave;
  const int nf32 = Nout / 32;
  const int ngroups = GATE_UP ? nf32 : nf32 / 2;
  if (g >= ngroups) return;  // no barriers in this kernel
  const int nk16 = K / 16;
  const uint16_t* base = GATE_UP
                             ? Bp + (size_t)(e * nf32 + g) * 2 * nk16 * kOperandElems
                             : Bp + (size_t)(e * nf32 + 2 * g) * nk16 * kOperandElems;
  const uint16_t* pb0 = base;
  const uint16_t* pb1 = base + (size_t)nk16 * kOperandElems;
  // 16x16x32 B operand from the 32x32x16 packed blocks: lane l takes column l%16 (+16 for
  // the second half), reduction rows 8*(l/16) .. + 8 of the 32-row k-step.
  const int ksub = lane >> 5;
  const int lofs = ((lane & 15) + 32 * ((lane >> 4) & 1)) * 8;
  const int nks = K / 32;

  for (int m0 = 0; m0 < cnt; m0 += 16) {
    f32x4_t acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = f32x4_t{};
    const int ar = row_beg + min(m0 + (lane & 15), cnt - 1);
    const uint16_t* ap = A + (size_t)ar * K + 8 * (lane >> 4);
#pragma unroll 4
    for (int ks = 0; ks < nks; ++ks) {
      const uint4 av = *(const uint4*)(ap + ks * 32);
      const size_t o = (size_t)(2 * ks + ksub) * kOperandElems + lofs;
      const uint4 v0 = *(const uint4*)(pb0 + o);
      const uint4 v1 = *(const uint4*)(pb0 + o + 16 * 8);
      const uint4 v2 = *(const uint4*)(pb1 + o);
      const uint4 v3 = *(const uint4*)(pb1 + o + 16 * 8);
      const bf16x8_t a = as_bf16x8(av);
      acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(v0), acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(v1), acc[1], 0, 0, 0);
      acc[2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(v2), acc[2], 0, 0, 0);
      acc[3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(v3), acc[3], 0, 0, 0);
    }
    // 16x16 accumulator layout: element i of lane l is row 4*(l/16) + i, column l%16.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m0 + 4 * (lane >> 4) + i;
      if (r >= cnt) continue;
      uint16_t* o = out + (size_t)(row_beg + r) * Nout;
      if (GATE_UP) {
        const int c = g * 32 + (lane & 15);
        o[c] = to_bf16(silu_mul(acc[0][i], acc[2][i]));
        o[c + 16] = to_bf16(silu_mul(acc[1][i], acc[3][i]));
      } else {
        const int c = g * 64 + (lane & 15);
        o[c] = to_bf16(acc[0][i]);
        o[c + 16] = to_bf16(acc[1][i]);
        o[c + 32] = to_bf16(acc[2][i]);
        o[c + 48] = to_bf16(acc[3][i]);
      }
    }
  }
}

}  // namespace

// Decode shape: few rows per expert on average.
bool ffn_use_decode(const moe_problem& p) { return (int64_t)p.T * p.k <= (int64_t)24 * p.E; }

hipError_t launch_tile_table(const moe_problem& p, const int32_t* offsets, TileTable tt,
                             hipStream_t s) {
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, s, offsets, p.E, tt.tile_count,
                     tt.tile_expert, tt.tile_row0);
  return hipGetLastError();
}

hipError_t launch_gate_up_bf16(const moe_problem& p, const void* xp, const int32_t* offsets,
                               const void* packed_gu, void* a, TileTable tt, hipStream_t s) {
  const int nf32 = p.I / 32;
  if (ffn_use_decode(p)) {
    hipLaunchKernelGGL(decode_kernel<true>, dim3(div_up(nf32, 4), p.E), dim3(256), 0, s,
                       (const uint16_t*)xp, offsets, (const uint16_t*)packed_gu, (uint16_t*)a,
                       p.H, p.I);
  } else {
    const int ntn = div_up(nf32, 8);
    hipLaunchKernelGGL(prefill_kernel<true>, dim3(ntn * tt.max_tiles), dim3(512), 0, s,
                       (const uint16_t*)xp, offsets, tt.tile_count, tt.tile_expert,
                       tt.tile_row0, (const uint16_t*)packed_gu, (uint16_t*)a, p.H, p.I, ntn);
  }
  return hipGetLastError();
}

hipError_t launch_down_bf16(const moe_problem& p, const void* a, const int32_t* offsets,
                            const void* packed_d, void* yp, TileTable tt, hipStream_t s) {
  const int nf32 = p.H / 32;
  if (ffn_use_decode(p)) {
    hipLaunchKernelGGL(decode_kernel<false>, dim3(div_up(nf32 / 2, 4), p.E), dim3(256), 0, s,
                       (const uint16_t*)a, offsets, (const uint16_t*)packed_d, (uint16_t*)yp,
                       p.I, p.H);
  } else {
    const int ntn = div_up(nf32, 16);
    hipLaunchKernelGGL(prefill_kernel<false>, dim3(ntn * tt.max_tiles), dim3(512), 0, s,
                       (const uint16_t*)a, offsets, tt.tile_count, tt.tile_expert,
                       tt.tile_row0, (const uint16_t*)packed_d, (uint16_t*)yp, p.I, p.H, ntn);
  }
  return hipGetLastError();
}

}  // namespace moe
