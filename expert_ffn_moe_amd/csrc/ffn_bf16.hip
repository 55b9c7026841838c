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
// Work item = (M tile of up to 256 rows of one expert, N group).  Wavefront w computes
// all rows of the tile for 2 operand columns (64 GEMM columns):
//   GATE_UP: the gate and the up column of 32 outputs of `a` -> block: 128 columns of a
//   DOWN   : 64 columns of yp                               -> block: 256 columns of yp
// 8 x 2 accumulators of 32x32 (256 fp32 per lane, in AGPRs); 32-row fragments past the
// expert's last row are skipped, so a ragged tile costs at most 31 idle rows.
//
// K runs in k-steps of 16 (one MFMA) grouped in stages of two.  Weight operands come
// straight from memory into a ring of 8 k-steps of registers (refilled as soon as a
// k-step's MFMAs are issued).  The 256x32 activation stage goes through LDS (double
// buffer, operand order, one contiguous 1 KiB fragment per wavefront store) and is
// loaded into registers 3 stages ahead.  Every wait therefore covers loads issued at
// least 3 stages earlier, although vector-memory counters complete in issue order.
//
// Scheduling: every block first turns `offsets` into per-expert M-tile starts (LDS).  The
// M tiles are split into 8 contiguous ranges, one per XCD (workgroups are dispatched to
// XCDs round-robin, so block b runs on XCD b % 8); the blocks of an XCD take its work
// items in turn.  Items of one expert therefore run together on one XCD, and the weight
// and activation bytes they share are served by that XCD's L2.
// ------------------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int kMaxExperts = 1024;
constexpr int kRing = 8;  // weight ring depth in k-steps

struct TileArgs {
  const uint16_t* A;     // activation rows of the tile (row0), row stride K
  const uint16_t* b0;    // first operand column of this wavefront (lane offset applied)
  const uint16_t* b1;    // second operand column
  uint16_t* out;         // output row row0, column col0 (row stride Nout)
  int K, Nout, rows, wave, lane, act;
};

// One step of the k loop: MFMAs of k-step (2 * stage + KK) from LDS buffer BUF and ring
// slot SLOT, then the ring slot is refilled with the operands KRING k-steps ahead.
template <int NM, int BUF, int KK, int SLOT>
__device__ __forceinline__ void kstep(f32x16_t (&acc)[8][2], uint4 (&bring)[kRing][2],
                                      const uint4 (*lds)[16 * 64], const TileArgs& t,
                                      int j_next) {
  bf16x8_t a[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) a[m] = as_bf16x8(lds[BUF][(m * 2 + KK) * 64 + t.lane]);
  const bf16x8_t bv0 = as_bf16x8(bring[SLOT][0]);
  const bf16x8_t bv1 = as_bf16x8(bring[SLOT][1]);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], bv0, acc[m][0], 0, 0, 0);
    acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], bv1, acc[m][1], 0, 0, 0);
  }
  const size_t o = (size_t)j_next * kOperandElems;
  bring[SLOT][0] = *(const uint4*)(t.b0 + o);
  bring[SLOT][1] = *(const uint4*)(t.b1 + o);
  __builtin_amdgcn_sched_barrier(0);
}

// One stage (two k-steps) with stage index s; U = s mod 4 picks registers and buffers.
template <int NM, int U>
__device__ __forceinline__ void kstage(f32x16_t (&acc)[8][2], uint4 (&bring)[kRing][2],
                                       uint4 (&aset)[4][4], uint4 (*lds)[16 * 64],
                                       const uint16_t* const (&ag)[4], const int (&lslot)[4],
                                       bool (&aload)[4], const TileArgs& t, int s, int nst,
                                       int nk16) {
  const int sa = min(s + 3, nst - 1);
#pragma unroll
  for (int p = 0; p < 4; ++p)
    if (aload[p]) aset[(U + 3) & 3][p] = *(const uint4*)(ag[p] + (size_t)sa * 32);
  __builtin_amdgcn_sched_barrier(0);
  kstep<NM, U & 1, 0, (2 * U) & 7>(acc, bring, lds, t, min(2 * s + kRing, nk16 - 1));
  kstep<NM, U & 1, 1, (2 * U + 1) & 7>(acc, bring, lds, t, min(2 * s + 1 + kRing, nk16 - 1));
#pragma unroll
  for (int p = 0; p < 4; ++p) lds[(U + 1) & 1][lslot[p]] = aset[(U + 1) & 3][p];
  __syncthreads();
}

// A whole work item with NM live 32-row fragments (NM = 2, 4, 6 or 8).
template <bool GATE_UP, int NM>
__device__ __forceinline__ void prefill_tile(const TileArgs& t, uint4 (*lds)[16 * 64]) {
  const int nk16 = t.K / 16, nst = t.K / 32;
  const int lane = t.lane, wave = t.wave;
  // activation loader: wavefront w fills fragments (m32 = 2w + p/2, k16 = p%2); lane L
  // takes row 32*m32 + L%32, k-offset 16*(p%2) + 8*(L/32): one contiguous LDS store each
  const uint16_t* ag[4];
  int lslot[4];
  bool aload[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int mf = 2 * wave + (p >> 1), kf = p & 1;
    const int r = mf * 32 + (lane & 31);
    ag[p] = t.A + (size_t)min(r, t.rows - 1) * t.K + kf * 16 + (lane >> 5) * 8;
    lslot[p] = (mf * 2 + kf) * 64 + lane;
    aload[p] = mf < NM;
  }
  f32x16_t acc[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m][0] = acc[m][1] = f32x16_t{};
  uint4 aset[4][4];
  uint4 bring[kRing][2];
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int st = min(u, nst - 1);
#pragma unroll
    for (int p = 0; p < 4; ++p)
      aset[u][p] = aload[p] ? *(const uint4*)(ag[p] + (size_t)st * 32) : uint4{0, 0, 0, 0};
  }
  aset[3][0] = aset[3][1] = aset[3][2] = aset[3][3] = uint4{0, 0, 0, 0};
#pragma unroll
  for (int q = 0; q < kRing; ++q) {
    const size_t o = (size_t)min(q, nk16 - 1) * kOperandElems;
    bring[q][0] = *(const uint4*)(t.b0 + o);
    bring[q][1] = *(const uint4*)(t.b1 + o);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) lds[0][lslot[p]] = aset[0][p];
  __syncthreads();
  for (int s0 = 0; s0 < nst; s0 += 4) {
    kstage<NM, 0>(acc, bring, aset, lds, ag, lslot, aload, t, s0, nst, nk16);
    if (s0 + 1 < nst) kstage<NM, 1>(acc, bring, aset, lds, ag, lslot, aload, t, s0 + 1, nst, nk16);
    if (s0 + 2 < nst) kstage<NM, 2>(acc, bring, aset, lds, ag, lslot, aload, t, s0 + 2, nst, nk16);
    if (s0 + 3 < nst) kstage<NM, 3>(acc, bring, aset, lds, ag, lslot, aload, t, s0 + 3, nst, nk16);
  }

  // Epilogue through LDS: per 32-row fragment, each wavefront writes its 32 x 32
  // (gate/up, after SwiGLU) or 32 x 64 (down) bf16 block row-major into its own 4 KiB of
  // LDS, then stores whole 16-byte row pieces.
  // 32x32 accumulator layout: element i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32.
  uint16_t* stage_out = reinterpret_cast<uint16_t*>(&lds[0][0]) + wave * 2048;
  constexpr int ncol = GATE_UP ? 32 : 64;
  constexpr int chunks = 32 * ncol / 8;  // 16-byte pieces per wavefront and fragment
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    if (m * 32 >= t.rows) break;  // block-uniform
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rr = (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
      if (GATE_UP) {
        stage_out[rr * ncol + (lane & 31)] = to_bf16(silu_mul(acc[m][0][i], acc[m][1][i]));
      } else {
        stage_out[rr * ncol + (lane & 31)] = to_bf16(acc[m][0][i]);
        stage_out[rr * ncol + 32 + (lane & 31)] = to_bf16(acc[m][1][i]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int q0 = 0; q0 < chunks; q0 += 64) {
      const int q = q0 + lane;
      const int rr = q / (ncol / 8), cc = q % (ncol / 8);
      const int r = m * 32 + rr;
      if (t.act && r < t.rows)
        *(uint4*)(t.out + (size_t)r * t.Nout + cc * 8) = *(const uint4*)(stage_out + rr * ncol + cc * 8);
    }
    __syncthreads();
  }
}

template <bool GATE_UP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ offsets, int E,
                    const uint16_t* __restrict__ Bp, uint16_t* __restrict__ out, int K, int Nout) {
  __shared__ uint4 lds_a[2][16 * 64];  // [buf][(m32 * 2 + k16) * 64 + lane]
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_wsum[4];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  // ---- per-expert M-tile starts (exclusive scan of ceil(count / 256))
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
  const int ntn = GATE_UP ? div_up(nf32, 4) : div_up(nf32, 8);
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int mt_lo = (int)((int64_t)total_mt * xcd / kXcds);
  const int mt_hi = (int)((int64_t)total_mt * (xcd + 1) / kXcds);
  const int items = (mt_hi - mt_lo) * ntn;
  const size_t panel = (size_t)nk16 * kOperandElems;

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
    TileArgs t;
    t.rows = min(kPrefillBM, offsets[e + 1] - row0);
    t.K = K;
    t.Nout = Nout;
    t.wave = wave;
    t.lane = lane;
    int col0;
    if (GATE_UP) {
      int af = nt * 4 + wave;
      t.act = af < nf32;
      af = min(af, nf32 - 1);
      t.b0 = Bp + (size_t)(e * nf32 + af) * 2 * panel;  // gate; up follows one panel later
      col0 = af * 32;
    } else {
      int nf = (nt * 4 + wave) * 2;
      t.act = nf < nf32;
      nf = min(nf, nf32 - 2);
      t.b0 = Bp + (size_t)(e * nf32 + nf) * panel;  // second column one panel later
      col0 = nf * 32;
    }
    t.b0 += lane * 8;
    t.b1 = t.b0 + panel;
    t.A = A + (size_t)row0 * K;
    t.out = out + (size_t)row0 * Nout + col0;
    const int nm = div_up(t.rows, 32);
    if (nm > 6) prefill_tile<GATE_UP, 8>(t, lds_a);
    else if (nm > 4) prefill_tile<GATE_UP, 6>(t, lds_a);
    else if (nm > 2) prefill_tile<GATE_UP, 4>(t, lds_a);
    else prefill_tile<GATE_UP, 2>(t, lds_a);
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
