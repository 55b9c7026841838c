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
//  * prefill (many rows per expert): persistent, XCD-aware grouped GEMM over 128-row M
//    tiles; the activation tile goes through LDS (shared by the 4 wavefronts of a block)
//    and each wavefront streams its own weight operands straight into registers in
//    matrix-core operand order (the packed layout makes each operand a contiguous 1 KiB).
//    v_mfma_f32_32x32x16_bf16.
//  * decode (a few rows per expert): a weight-streaming kernel; one wavefront per
//    32/64-column panel of one expert, 16-row M steps, v_mfma_f32_16x16x32_bf16.
#include <algorithm>

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
// Prefill grouped GEMM: persistent, one block of 4 wavefronts per CU.
//
// Work item = (M tile of 128 rows of one expert, N group).  Wavefront w of the block
// computes 128 rows x 4 operand columns (4 x 32 = 128 GEMM columns):
//   GATE_UP: gate and up columns of 64 outputs of `a` -> block covers 256 columns of a
//   DOWN   : 128 columns of yp                          -> block covers 512 columns of yp
// 16 accumulators of 32x32 (256 fp32 registers per lane, held in AGPRs).
//
// K runs in stages of 64 (4 MFMA k-steps).  The 128x64 activation stage goes through LDS
// (double-buffered, matrix-core operand order, shared by the 4 wavefronts); each
// wavefront's weight operands come straight from memory into registers, one stage ahead.
//
// Scheduling: every block first turns `offsets` into per-expert M-tile starts (LDS).  The
// M tiles are split into 8 contiguous ranges, one per XCD (workgroups are dispatched to
// XCDs round-robin, so block b runs on XCD b % 8); the blocks of an XCD take its work
// items in turn.  Items of one expert therefore run together on one XCD, and the weight
// and activation bytes they share are served by that XCD's L2.
// ------------------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int kMaxExperts = 1024;

template <bool GATE_UP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int E,
                    const uint16_t* __restrict__ Bp, uint16_t* __restrict__ out, int K, int Nout) {
  __shared__ uint4 lds_a[2][16 * 64];  // [buf][(m32 * 4 + k16) * 64 + lane]
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_wsum[4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  // ---- per-expert M-tile starts (exclusive scan of ceil(count / 128))
  {
    const int per = div_up(E, 256);
    const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
    int sum = 0;
    for (int e = e0; e < e1; ++e) sum += div_up(offsets[e + 1] - offsets[e], kPrefillBM);
    const int inc = wave_inclusive_scan(sum);
    if (lane == 63) s_wsum[wave] = inc;
    __syncthreads();
    int base = inc - sum;
    for (int w = 0; w < wave; ++w) base += s_wsum[w];
    for (int e = e0; e < e1; ++e) {
      s_start[e] = base;
      base += div_up(offsets[e + 1] - offsets[e], kPrefillBM);
    }
    if (tid == 255) s_start[E] = base;
    __syncthreads();
  }
  const int total_mt = s_start[E];
  const int nk16 = K / 16;
  const int nf32 = Nout / 32;
  const int ntn = GATE_UP ? div_up(nf32, 8) : div_up(nf32, 16);
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int mt_lo = (int)((int64_t)total_mt * xcd / kXcds);
  const int mt_hi = (int)((int64_t)total_mt * (xcd + 1) / kXcds);
  const int items = (mt_hi - mt_lo) * ntn;
  const int nst = K / 64;

  for (int item = slot; item < items; item += nslots) {
    const int mt = mt_lo + item / ntn;
    const int nt = item - (item / ntn) * ntn;
    // expert of tile mt: the largest e with s_start[e] <= mt
    int lo = 0, hi = E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_start[mid] <= mt) lo = mid; else hi = mid;
    }
    const int e = lo;
    const int row0 = offsets[e] + (mt - s_start[e]) * kPrefillBM;
    const int rows = min(kPrefillBM, offsets[e + 1] - row0);

    // this wavefront's 4 operand columns
    const uint16_t* bs[4];
    int fcol[4];
    bool act[4];
    const size_t panel = (size_t)nk16 * kOperandElems;
    if (GATE_UP) {
      int af0 = (nt * 4 + wave) * 2;  // two 32-column groups of `a`
      act[0] = act[1] = act[2] = act[3] = af0 < nf32;
      af0 = min(af0, nf32 - 2);
      const uint16_t* g0 = Bp + (size_t)(e * nf32 + af0) * 2 * panel;
      bs[0] = g0;              // gate, columns af0
      bs[1] = g0 + 2 * panel;  // gate, columns af0 + 1
      bs[2] = g0 + panel;      // up,   columns af0
      bs[3] = g0 + 3 * panel;  // up,   columns af0 + 1
      fcol[0] = fcol[2] = af0 * 32;
      fcol[1] = fcol[3] = af0 * 32 + 32;
    } else {
      const int nf0 = (nt * 4 + wave) * 4;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        act[c] = nf0 + c < nf32;
        const int f = min(nf0 + c, nf32 - 1);
        bs[c] = Bp + (size_t)(e * nf32 + f) * panel;
        fcol[c] = f * 32;
      }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) bs[c] += lane * 8;

    // activation stage loader: wavefront w fills the 4 operand fragments of rows
    // 32w .. 32w+31 (one per k-step); lane L of the p-th load takes row 32w + L%32,
    // k-offset 16p + 8*(L/32), so every LDS write is one contiguous 1 KiB fragment.
    const uint16_t* ag[4];
    int lslot[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = wave * 32 + (lane & 31);
      ag[p] = A + (size_t)(row0 + min(r, rows - 1)) * K + p * 16 + (lane >> 5) * 8;
      lslot[p] = (wave * 4 + p) * 64 + lane;
    }

    f32x16_t acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[m][c] = f32x16_t{};

    // b[kk][c]: operand column c of k-step kk of the current stage.  Each k-step's
    // registers are refilled with the next stage's operands as soon as its MFMAs are
    // issued, so a load has a whole stage (16 MFMAs x 4 k-steps) to land.
    uint4 areg[4], b[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) areg[p] = *(const uint4*)(ag[p]);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int c = 0; c < 4; ++c) b[kk][c] = *(const uint4*)(bs[c] + (size_t)kk * kOperandElems);
#pragma unroll
    for (int p = 0; p < 4; ++p) lds_a[0][lslot[p]] = areg[p];
    __syncthreads();

    for (int st = 0; st < nst; ++st) {
      const int cur = st & 1;
      // Next stage's operands.  The loads are unconditional (the last stage reloads
      // itself, into registers and a buffer nobody reads) so that the compiler cannot
      // merge the load and the LDS store behind one branch and wait on the load at once.
      const int sn = min(st + 1, nst - 1);
#pragma unroll
      for (int p = 0; p < 4; ++p) areg[p] = *(const uint4*)(ag[p] + (size_t)sn * 64);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t a[4], an[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) a[m] = as_bf16x8(lds_a[cur][(m * 4 + 0) * 64 + lane]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        // the next k-step's activation fragments are read before this k-step's MFMAs
        if (kk < 3) {
#pragma unroll
          for (int m = 0; m < 4; ++m) an[m] = as_bf16x8(lds_a[cur][(m * 4 + kk + 1) * 64 + lane]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8_t bv = as_bf16x8(b[kk][c]);
#pragma unroll
          for (int m = 0; m < 4; ++m)
            acc[m][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], bv, acc[m][c], 0, 0, 0);
        }
        const size_t o = (size_t)(sn * 4 + kk) * kOperandElems;
#pragma unroll
        for (int c = 0; c < 4; ++c) b[kk][c] = *(const uint4*)(bs[c] + o);
        if (kk < 3) {
#pragma unroll
          for (int m = 0; m < 4; ++m) a[m] = an[m];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) lds_a[cur ^ 1][lslot[p]] = areg[p];
      __syncthreads();
    }

    // 32x32 accumulator layout: element i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
    // column l%32.
    const int lc = lane & 31;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = m * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (r >= rows) continue;
        uint16_t* o = out + (size_t)(row0 + r) * Nout + lc;
        if (GATE_UP) {
          if (act[0]) {
            o[fcol[0]] = to_bf16(silu_mul(acc[m][0][i], acc[m][2][i]));
            o[fcol[1]] = to_bf16(silu_mul(acc[m][1][i], acc[m][3][i]));
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (act[c]) o[fcol[c]] = to_bf16(acc[m][c][i]);
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

namespace {
int cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}
int persistent_grid() { return std::max(kXcds, cu_count() / kXcds * kXcds); }
}  // namespace

hipError_t launch_gate_up_bf16(const moe_problem& p, const void* xp, const int32_t* offsets,
                               const void* packed_gu, void* a, hipStream_t s) {
  if (ffn_use_decode(p)) {
    const int nf32 = p.I / 32;
    hipLaunchKernelGGL(decode_kernel<true>, dim3(div_up(nf32, 4), p.E), dim3(256), 0, s,
                       (const uint16_t*)xp, offsets, (const uint16_t*)packed_gu, (uint16_t*)a,
                       p.H, p.I);
  } else {
    hipLaunchKernelGGL(prefill_kernel<true>, dim3(persistent_grid()), dim3(256), 0, s,
                       (const uint16_t*)xp, offsets, p.E, (const uint16_t*)packed_gu,
                       (uint16_t*)a, p.H, p.I);
  }
  return hipGetLastError();
}

hipError_t launch_down_bf16(const moe_problem& p, const void* a, const int32_t* offsets,
                            const void* packed_d, void* yp, hipStream_t s) {
  if (ffn_use_decode(p)) {
    const int nf32 = p.H / 32;
    hipLaunchKernelGGL(decode_kernel<false>, dim3(div_up(nf32 / 2, 4), p.E), dim3(256), 0, s,
                       (const uint16_t*)a, offsets, (const uint16_t*)packed_d, (uint16_t*)yp,
                       p.I, p.H);
  } else {
    hipLaunchKernelGGL(prefill_kernel<false>, dim3(persistent_grid()), dim3(256), 0, s,
                       (const uint16_t*)a, offsets, p.E, (const uint16_t*)packed_d,
                       (uint16_t*)yp, p.I, p.H);
  }
  return hipGetLastError();
}

}  // namespace moe
