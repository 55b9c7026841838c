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
//    tiles; the activation tile goes through LDS (shared by the 8 wavefronts of a block)
//    and each wavefront streams its own weight operands straight into registers in
//    matrix-core operand order (the packed layout makes each operand a contiguous 1 KiB).
//    v_mfma_f32_32x32x16_bf16.  The same tile computes the backward pass's weight
//    gradients (wgrad_kernel).
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

constexpr int kOperandElems = 512;  // one packed 32x16 (or 16x32) operand block

constexpr int kXcds = 8;
constexpr int kMaxExperts = 1024;
constexpr int kWaves = 8;               // wavefronts per block (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kRing = 4;                // weight ring depth in k-steps (one stage)

struct TileArgs {
  const uint16_t* A;     // activation row row0 of the tile, row stride K (with a row
                         // gather: the token rows x, row i of the tile being rtok[i])
  const int32_t* rtok;   // row gather only: row_token + row0
  const uint16_t* b0;    // this wavefront's first operand column (lane offset applied)
  const uint16_t* b1;    // second operand column
  uint16_t* out;         // output row row0, column col0 (row stride Nout)
  uint16_t* out2;        // gate/up saving g|u: that row of gu, column 2 col0 (row stride 2 Nout)
  float* outf;           // weight gradients: fp32 output row row0, column col0
  float* outf2;          // ... its up half when the columns are the interleaved gate|up
  int K, Nout, rows, wave, lane, act;
  int nst;               // stages of 64 along K
  int col0;              // weight gradients: the wavefront's first output column
  int gu_split;
  int fbase[4];          // LDS index of this lane's fragment piece, per k-step, m32 = 0
};

// Tile epilogues: SwiGLU to bf16 `a`, bf16 GEMM output, fp32 weight gradient.
enum TileMode { kModeGateUp = 0, kModeDown = 1, kModeWgrad = 2 };

// LDS activation stage: 128 rows x 64 k bf16, row-major, 16-byte chunk c of row r stored
// at chunk position c ^ f(r), f(r) = ((r >> 1) ^ (r << 2)) & 7.  f takes 8 distinct values
// on any 8 consecutive rows and on the even (and the odd) rows of any 16, so a wavefront
// store of 8 rows x 8 chunks and a fragment read of 32 rows x 1 chunk are free of bank
// conflicts whether the LDS serves 8 or 16 lanes of 16-byte accesses per cycle.  f depends
// on r mod 16 only: a lane's fragment piece for 32-row group m sits at
// fbase[k-step] + 256 * m (uint4 units), and stage buffer b adds 1024 * b.
__device__ __forceinline__ int a_slot(int r, int c) {
  return r * 8 + (c ^ (((r >> 1) ^ (r << 2)) & 7));
}

// k-step KK of a stage: MFMAs with activation fragments `a` and ring slot KK, then the
// slot is refilled with operand k-step j_next; the next k-step's fragments are read
// from LDS first so that their latency hides behind these MFMAs.
template <int NM, int BUF, int KK>
__device__ __forceinline__ void kstep(f32x16_t (&acc)[4][2], u32x4 (&bring)[kRing][2],
                                      bf16x8_t (&a)[4], const u32x4 (*lds)[1024],
                                      const TileArgs& t, int j_next) {
  bf16x8_t an[4];
  if (KK < 3) {
    const u32x4* base = &lds[BUF][0] + t.fbase[KK + 1];
#pragma unroll
    for (int m = 0; m < NM; ++m) an[m] = as_bf16x8(base[256 * m]);
  }
  __builtin_amdgcn_sched_barrier(0);
  const bf16x8_t bv0 = as_bf16x8(bring[KK][0]);
  const bf16x8_t bv1 = as_bf16x8(bring[KK][1]);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], bv0, acc[m][0], 0, 0, 0);
    acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m], bv1, acc[m][1], 0, 0, 0);
  }
  const size_t o = (size_t)j_next * kOperandElems;
  bring[KK][0] = *(const u32x4*)(t.b0 + o);
  bring[KK][1] = *(const u32x4*)(t.b1 + o);
  if (KK < 3) {
#pragma unroll
    for (int m = 0; m < NM; ++m) a[m] = an[m];
  }
  __builtin_amdgcn_sched_barrier(0);
}

// One stage (4 k-steps of 16) from LDS buffer BUF.  Activations are loaded two stages
// ahead into register set BUF and stored to LDS one stage ahead.
template <int NM, int BUF>
__device__ __forceinline__ void kstage(f32x16_t (&acc)[4][2], u32x4 (&bring)[kRing][2],
                                       u32x4 (&aset0)[2], u32x4 (&aset1)[2],
                                       u32x4 (*lds)[1024], const uint16_t* const (&ag)[2],
                                       const int (&lslot)[2], const TileArgs& t, int s,
                                       int nst) {
  const size_t sa = (size_t)min(s + 2, nst - 1) * 64;
  if constexpr (BUF == 0) {
    aset0[0] = *(const u32x4*)(ag[0] + sa);
    aset0[1] = *(const u32x4*)(ag[1] + sa);
  } else {
    aset1[0] = *(const u32x4*)(ag[0] + sa);
    aset1[1] = *(const u32x4*)(ag[1] + sa);
  }
  __builtin_amdgcn_sched_barrier(0);
  bf16x8_t a[4];
  {
    const u32x4* base = &lds[BUF][0] + t.fbase[0];
#pragma unroll
    for (int m = 0; m < NM; ++m) a[m] = as_bf16x8(base[256 * m]);
  }
  // ring slots are refilled with the next stage's operands
  const int jn = 4 * (s + 1), jmax = 4 * nst - 1;
  kstep<NM, BUF, 0>(acc, bring, a, lds, t, min(jn + 0, jmax));
  kstep<NM, BUF, 1>(acc, bring, a, lds, t, min(jn + 1, jmax));
  kstep<NM, BUF, 2>(acc, bring, a, lds, t, min(jn + 2, jmax));
  kstep<NM, BUF, 3>(acc, bring, a, lds, t, min(jn + 3, jmax));
  // stage s + 1 (loaded at the start of stage s - 1) into the other buffer
  if constexpr (BUF == 0) {
    lds[1][lslot[0]] = aset1[0];
    lds[1][lslot[1]] = aset1[1];
  } else {
    lds[0][lslot[0]] = aset0[0];
    lds[0][lslot[1]] = aset0[1];
  }
  __syncthreads();
}

// One work item: 128 rows x (this wavefront's two operand columns), t.nst >= 1 stages.
template <int MODE, bool GATHER, bool SAVE_GU = false>
__device__ __forceinline__ void prefill_tile(const TileArgs& t, u32x4 (*lds)[1024]) {
  constexpr bool GATE_UP = MODE == kModeGateUp;
  const int nst = t.nst;
  const int lane = t.lane, wave = t.wave;
  // activation loader: the p-th load of wavefront w covers rows 64p + 8w .. + 7, lane L
  // taking chunk L % 8 of row L / 8: whole 128-byte lines
  const uint16_t* ag[2];
  int lslot[2];
  const int lr = wave * 8 + (lane >> 3), lc = lane & 7;
  const int lbase = a_slot(lr, lc);  // rows 64p + lr share f(r): slot lbase + 512p
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int r = min(p * 64 + lr, t.rows - 1);
    const size_t src_row = GATHER ? (size_t)t.rtok[r] : (size_t)r;
    ag[p] = t.A + src_row * t.K + lc * 8;
    lslot[p] = lbase + 512 * p;
  }
  f32x16_t acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m][0] = acc[m][1] = f32x16_t{};
  u32x4 aset0[2], aset1[2];
  u32x4 bring[kRing][2];
  const size_t s1 = (size_t)min(1, nst - 1) * 64;
  aset0[0] = *(const u32x4*)(ag[0]);
  aset0[1] = *(const u32x4*)(ag[1]);
  aset1[0] = *(const u32x4*)(ag[0] + s1);
  aset1[1] = *(const u32x4*)(ag[1] + s1);
#pragma unroll
  for (int q = 0; q < kRing; ++q) {
    const size_t o = (size_t)min(q, 4 * nst - 1) * kOperandElems;
    bring[q][0] = *(const u32x4*)(t.b0 + o);
    bring[q][1] = *(const u32x4*)(t.b1 + o);
  }
  lds[0][lslot[0]] = aset0[0];
  lds[0][lslot[1]] = aset0[1];
  __syncthreads();
  if (t.rows > 64) {  // block-uniform: a tile with at most 64 (32) live rows skips the others
    // stages in pairs with an odd last stage peeled off: with the second stage of a pair
    // conditional, the compiler sank the first stage's activation loads into it (their
    // only use), leaving them one stage of latency instead of two
    int s0 = 0;
    for (; s0 + 1 < nst; s0 += 2) {
      kstage<4, 0>(acc, bring, aset0, aset1, lds, ag, lslot, t, s0, nst);
      kstage<4, 1>(acc, bring, aset0, aset1, lds, ag, lslot, t, s0 + 1, nst);
    }
    if (s0 < nst) kstage<4, 0>(acc, bring, aset0, aset1, lds, ag, lslot, t, s0, nst);
  } else if (t.rows > 32) {  // 64 rows (the last tile of an expert, mostly)
    int s0 = 0;
    for (; s0 + 1 < nst; s0 += 2) {
      kstage<2, 0>(acc, bring, aset0, aset1, lds, ag, lslot, t, s0, nst);
      kstage<2, 1>(acc, bring, aset0, aset1, lds, ag, lslot, t, s0 + 1, nst);
    }
    if (s0 < nst) kstage<2, 0>(acc, bring, aset0, aset1, lds, ag, lslot, t, s0, nst);
  } else {  // 32 rows: measured 1.5-3% faster GEMMs on the prefill shapes than 64
    int s0 = 0;
    for (; s0 + 1 < nst; s0 += 2) {
      kstage<1, 0>(acc, bring, aset0, aset1, lds, ag, lslot, t, s0, nst);
      kstage<1, 1>(acc, bring, aset0, aset1, lds, ag, lslot, t, s0 + 1, nst);
    }
    if (s0 < nst) kstage<1, 0>(acc, bring, aset0, aset1, lds, ag, lslot, t, s0, nst);
  }

  if constexpr (MODE == kModeWgrad) {
    // fp32 through LDS: per (32-row fragment, operand column) the wavefront writes its
    // 32 x 32 block row-major into its own 4 KiB of LDS (a half wavefront writes one row
    // of 32 consecutive floats per register) and stores it in 16-byte pieces, 8 lanes per
    // 128-byte row piece, with the non-temporal hint (the gradients are written once and
    // are far larger than the caches).  The region is the wavefront's own and a
    // wavefront's LDS accesses complete in order, so the phases need only a compiler
    // barrier.
    if (!t.act) return;
    float* const ldsf = reinterpret_cast<float*>(&lds[0][0]) + wave * 1024;
    const int wofs = (lane >> 5) * 4 * 32 + (lane & 31);
    const int qrow = lane >> 3, qcol = (lane & 7) * 4;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (m * 32 >= t.rows) break;  // block-uniform
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int i = 0; i < 16; ++i) ldsf[wofs + ((i >> 2) * 8 + (i & 3)) * 32] = acc[m][h][i];
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        float* o;
        size_t ld;
        if (!t.gu_split) {
          o = t.outf + t.col0 + 32 * h;
          ld = t.Nout;
        } else {  // interleaved gate|up columns: operand column 0 -> gate, 1 -> up
          o = (h ? t.outf2 : t.outf) + 32 * (t.col0 >> 6);
          ld = t.Nout / 2;
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int rr = qrow + 8 * p, r = m * 32 + rr;
          const f32x4_t v = *(const f32x4_t*)(ldsf + rr * 32 + qcol);
          if (r < t.rows) __builtin_nontemporal_store(v, (f32x4_t*)(o + (size_t)r * ld + qcol));
        }
        __asm__ volatile("" ::: "memory");
      }
    }
    return;
  }

  // Epilogue through LDS: per 32-row fragment, each wavefront writes its 32 x 32 (gate/up,
  // after SwiGLU) or 32 x 64 (down) bf16 block row-major into its own 4 KiB of LDS, then
  // stores whole 16-byte row pieces.
  // 32x32 accumulator layout: element i of lane l is row 8*(i/4) + 4*(l/32) + i%4,
  // column l%32.
  constexpr int ncol = GATE_UP ? 32 : 64;
  constexpr int chunks = 32 * ncol / 8;  // 16-byte pieces per wavefront and fragment
  uint16_t* const lds16 = reinterpret_cast<uint16_t*>(&lds[0][0]) + wave * 2048;
  const int wofs = (lane >> 5) * 4 * ncol + (lane & 31);  // element (row 4*(l/32), col l%32)
  const int qrow = lane / (ncol / 8), qcol = (lane % (ncol / 8)) * 8;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m * 32 < t.rows) {  // block-uniform
      if constexpr (GATE_UP && SAVE_GU) {
        // the pre-activations first, as the plain GEMM over the same operand columns stores
        // them: a 32 x 64 block, the gate column's 32 values then the up column's
        const int wofs2 = (lane >> 5) * 4 * 64 + (lane & 31);
        const int qrow2 = lane >> 3, qcol2 = (lane & 7) * 8;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          uint16_t* srow = lds16 + wofs2 + ((i >> 2) * 8 + (i & 3)) * 64;
          srow[0] = to_bf16(acc[m][0][i]);
          srow[32] = to_bf16(acc[m][1][i]);
        }
        __syncthreads();
#pragma unroll
        for (int q0 = 0; q0 < 256; q0 += 64) {
          const int rr = qrow2 + q0 / 8;
          const int r = m * 32 + rr;
          if (t.act && r < t.rows)
            *(u32x4*)(t.out2 + (size_t)r * 2 * t.Nout + qcol2) =
                *(const u32x4*)(lds16 + rr * 64 + qcol2);
        }
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint16_t* srow = lds16 + wofs + ((i >> 2) * 8 + (i & 3)) * ncol;
        if (GATE_UP) {
          srow[0] = to_bf16(silu_mul(acc[m][0][i], acc[m][1][i]));
        } else {
          srow[0] = to_bf16(acc[m][0][i]);
          srow[32] = to_bf16(acc[m][1][i]);
        }
      }
      __syncthreads();
#pragma unroll
      for (int q0 = 0; q0 < chunks; q0 += 64) {
        const int rr = qrow + q0 / (ncol / 8);
        const int r = m * 32 + rr;
        if (t.act && r < t.rows)
          *(u32x4*)(t.out + (size_t)r * t.Nout + qcol) = *(const u32x4*)(lds16 + rr * ncol + qcol);
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------------------------
// Prefill grouped GEMM: persistent, one block of 8 wavefronts per CU.
//
// Work item = (M tile of 128 rows of one expert, N group).  Wavefront w computes the
// tile's 128 rows for 2 operand columns (64 GEMM columns):
//   GATE_UP: the gate and the up column of 32 outputs of `a` -> block: 256 columns of a
//   DOWN   : 64 columns of yp                               -> block: 512 columns of yp
// 4 x 2 accumulators of 32x32 (128 fp32 per lane, in AGPRs).
//
// K runs in stages of 64 (4 MFMA k-steps of 16).  The 128x64 activation stage goes
// through LDS (double buffer, XOR-swizzled rows, loaded as whole 128-byte lines two
// stages ahead); each wavefront's weight operands come straight from memory into a
// one-stage register ring (each k-step's slot refilled as soon as its MFMAs issue).
//
// Scheduling: every block first turns `offsets` into per-expert M-tile starts (LDS).  The
// M tiles are split into 8 contiguous ranges, one per XCD (workgroups are dispatched to
// XCDs round-robin, so block b runs on XCD b % 8); the blocks of an XCD take its work
// items in turn, expert by expert, and within an expert N group by N group with the M
// tiles innermost (measured 2-3.5% faster than M-tile-major on the three prefill shapes).
// Items of one expert therefore run together on one XCD, and the weight and activation
// bytes they share are served by that XCD's L2.  Without `claim` the blocks of an XCD take
// its items round-robin; with it (8 counters, zero at launch) a block's first item is its
// slot and each further item is claimed from its XCD's counter when the block starts the
// item before (the atomic's latency hides behind that item), so blocks that drew short
// tiles take more items: with only a few items per block (the smaller prefill shapes) the
// static split ends with some blocks idle while others still run.
// ------------------------------------------------------------------------------------
// GATHER (gate/up only): the activation rows are token rows x[row_token[r]] instead of
// xp[r], so the dispatch row copy is folded into this kernel's activation loads.
// SAVE_GU (gate/up only): the pre-activations g|u are stored too, into gu [rows, 2 Nout] in
// the layout (and with the bits) of the plain GEMM over the packed gate/up weights.
template <bool GATE_UP, bool GATHER, bool SAVE_GU = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ row_token,
                    const int32_t* __restrict__ offsets, int E,
                    const uint16_t* __restrict__ Bp, uint16_t* __restrict__ out, int K, int Nout,
                    uint16_t* __restrict__ gu, int* __restrict__ claim) {
  __shared__ u32x4 lds_a[2][1024];  // two activation stages (see a_slot)
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_wsum[kWaves];
  __shared__ int s_claim[2];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;

  // ---- per-expert M-tile starts (exclusive scan of ceil(count / 128))
  {
    const int per = div_up(E, kThreads);
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
    if (tid == kThreads - 1) s_start[E] = base;
    __syncthreads();
  }
  const int total_mt = s_start[E];
  const int nk16 = K / 16;
  const int nf32 = Nout / 32;
  const int ntn = GATE_UP ? div_up(nf32, kWaves) : div_up(nf32, 2 * kWaves);
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int mt_lo = (int)((int64_t)total_mt * xcd / kXcds);
  const int mt_hi = (int)((int64_t)total_mt * (xcd + 1) / kXcds);
  const int items = (mt_hi - mt_lo) * ntn;
  const size_t panel = (size_t)nk16 * kOperandElems;

  int cpar = 0;
  for (int item = slot; item < items;) {
    int claimed = 0;
    if (claim != nullptr && tid == 0)
      claimed = __hip_atomic_fetch_add(claim + xcd, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // The items of the range, expert by expert (its M tiles inside the range): N group
    // major, M tile minor.  The expert's segment of items starts at ntn times its first
    // tile's offset in the range, so the expert is that of tile mt_lo + item / ntn: the
    // largest e with s_start[e] <= that tile.
    int lo = 0, hi = E;
    {
      const int q = mt_lo + item / ntn;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_start[mid] <= q) lo = mid; else hi = mid;
      }
    }
    const int e = lo;
    const int seg0 = max(s_start[e], mt_lo), nte = min(s_start[e + 1], mt_hi) - seg0;
    const int local = item - ntn * (seg0 - mt_lo);
    const int nt = local / nte;
    const int mt = seg0 + (local - nt * nte);
    const int row0 = offsets[e] + (mt - s_start[e]) * kPrefillBM;
    TileArgs t;
    t.rows = min(kPrefillBM, offsets[e + 1] - row0);
    t.K = K;
    t.nst = K / 64;
    t.Nout = Nout;
    t.wave = wave;
    // lane goes through an empty asm statement so that nothing derived from it is
    // invariant across work items (the compiler would otherwise hoist the per-lane
    // addresses of the epilogue out of this loop and keep them live through the k loop)
    int lane_v = lane;
    __asm__ volatile("" : "+v"(lane_v));
    t.lane = lane_v;
    int col0;
    if (GATE_UP) {
      int af = nt * kWaves + wave;  // 32 columns of `a`: gate and up operand columns
      t.act = af < nf32;
      af = min(af, nf32 - 1);
      t.b0 = Bp + (size_t)(e * nf32 + af) * 2 * panel;
      t.b1 = t.b0 + panel;
      col0 = af * 32;
    } else {
      int nf = (nt * kWaves + wave) * 2;  // 64 columns of yp
      t.act = nf < nf32;
      nf = min(nf, nf32 - 2);
      t.b0 = Bp + (size_t)(e * nf32 + nf) * panel;
      t.b1 = t.b0 + panel;
      col0 = nf * 32;
    }
    t.b0 += lane_v * 8;
    t.b1 += lane_v * 8;
    t.A = GATHER ? A : A + (size_t)row0 * K;
    t.rtok = GATHER ? row_token + row0 : nullptr;
    t.out = out + (size_t)row0 * Nout + col0;
    t.out2 = SAVE_GU ? gu + (size_t)row0 * 2 * Nout + 2 * col0 : nullptr;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) t.fbase[kk] = a_slot(lane_v & 31, 2 * kk + (lane_v >> 5));
    prefill_tile<GATE_UP ? kModeGateUp : kModeDown, GATHER, SAVE_GU>(t, lds_a);
    if (claim != nullptr) {  // block-uniform
      // two LDS slots: the slot written here was last read before the previous barrier
      if (tid == 0) s_claim[cpar] = claimed;
      __syncthreads();
      item = nslots + s_claim[cpar];
      cpar ^= 1;
    } else {
      item += nslots;
    }
  }
}

// ------------------------------------------------------------------------------------
// Weight gradients of every expert (backward pass): out[e][m][n] = sum over the expert's
// rows k of AT[m][k] BT[n][k], with AT [M][npad] bf16 row-major and BT [Ncols][npad] in
// packed operand order (1 KiB blocks [n / 32][k / 16], like the packed down weights); each
// expert's rows padded with zeros to a multiple of 64 starting at poff[e].  The prefill
// tile with the roles of the forward: tile rows = 128 of M, a wavefront's two operand
// columns = 64 of Ncols (512 per block of 8 wavefronts), each k-step one contiguous 1 KiB
// operand block, K = the rows; fp32 out.  (With BT row-major, a k-step read 32 B of each of
// 32 rows per load and every 128-byte line was fetched four times from L2.)  gu_split: Ncols is the interleaved gate|up dimension, the columns go to out
// (gate) and out2 (up), each [E][M][Ncols / 2].  Grid: (M / 128 rounded up, Ncols / 512
// rounded up, E); experts without rows get zeros.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void wgrad_kernel(const uint16_t* __restrict__ AT, const uint16_t* __restrict__ BT,
                  const int32_t* __restrict__ poff, int M, int Ncols, int npad, int gu_split,
                  float* __restrict__ out, float* __restrict__ out2) {
  __shared__ u32x4 lds_a[2][1024];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int e = blockIdx.z;
  const int m0 = blockIdx.x * kPrefillBM;
  const int k0 = poff[e], kn = poff[e + 1] - k0;
  TileArgs t;
  t.rows = min(kPrefillBM, M - m0);
  t.K = npad;  // the A row stride
  t.nst = kn / 64;
  t.Nout = Ncols;
  t.wave = wave;
  t.lane = lane;
  const int n0 = blockIdx.y * 64 * kWaves + wave * 64;
  t.act = n0 < Ncols;
  const int nc = min(n0, Ncols - 64);  // idle wavefronts keep valid (unstored) columns
  t.col0 = nc;
  t.gu_split = gu_split;
  t.A = AT + (size_t)m0 * npad + k0;
  t.rtok = nullptr;
  t.b0 = BT + ((size_t)(nc >> 5) * (npad >> 4) + (k0 >> 4)) * kOperandElems + lane * 8;
  t.b1 = t.b0 + (size_t)(npad >> 4) * kOperandElems;  // the next 32 columns
  const size_t orow = (size_t)e * M + m0;
  t.outf = out + orow * (gu_split ? Ncols / 2 : Ncols);
  t.outf2 = gu_split ? out2 + orow * (Ncols / 2) : nullptr;
  t.out = nullptr;
  t.out2 = nullptr;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) t.fbase[kk] = a_slot(lane & 31, 2 * kk + (lane >> 5));
  if (t.nst > 0) {  // block-uniform
    prefill_tile<kModeWgrad, false>(t, lds_a);
    return;
  }
  if (!t.act) return;
  for (int r = 0; r < t.rows; ++r)
    for (int h = 0; h < 2; ++h) {
      const int n = nc + 32 * h + (lane & 31);
      if (lane >= 32) continue;
      if (!gu_split)
        t.outf[(size_t)r * Ncols + n] = 0.0f;
      else
        ((n & 32) ? t.outf2 : t.outf)[(size_t)r * (Ncols / 2) + 32 * (n >> 6) + (n & 31)] = 0.0f;
    }
}

// ------------------------------------------------------------------------------------
// Decode (weight streaming).  One wavefront per panel of one expert:
//   GATE_UP: 32 columns of `a` (gate + up operand columns): each k-step of 32 issues 4 B
//            operand loads (16 columns each) and one A load;
//   DOWN   : 32 columns of yp, two k-steps per iteration (the same 4 B loads in flight).
// The wavefronts hold few registers, so 32 of them share a CU; 32 columns each make the
// DSV3-shaped down projection 224 wavefronts per CU (7 full rounds; with 64 columns it was
// 3.5, the last round half empty).
// ------------------------------------------------------------------------------------
template <bool GATE_UP, bool GATHER, bool SAVE_GU = false>
__global__ __launch_bounds__(256) void decode_kernel(const uint16_t* __restrict__ A,
                                                     const int32_t* __restrict__ row_token,
                                                     const int32_t* __restrict__ offsets,
                                                     const uint16_t* __restrict__ Bp,
                                                     uint16_t* __restrict__ out, int K,
                                                     int Nout,
                                                     uint16_t* __restrict__ gu) {
  const int e = blockIdx.y;
  const int row_beg = offsets[e];
  const int cnt = offsets[e + 1] - row_beg;
  if (cnt <= 0) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = blockIdx.x * 4 + wave;
  const int nf32 = Nout / 32;
  const int ngroups = nf32;
  if (g >= ngroups) return;  // no barriers in this kernel
  const int nk16 = K / 16;
  const uint16_t* base = GATE_UP
                             ? Bp + (size_t)(e * nf32 + g) * 2 * nk16 * kOperandElems
                             : Bp + (size_t)(e * nf32 + g) * nk16 * kOperandElems;
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
    const size_t src_row = GATHER ? (size_t)row_token[ar] : (size_t)ar;
    const uint16_t* ap = A + src_row * K + 8 * (lane >> 4);
    // weights are read once per launch: non-temporal loads (measured 5-7% faster on
    // 7168 x 2048 experts than cached loads)
    if constexpr (GATE_UP) {
      for (int ks = 0; ks < nks; ++ks) {
        const uint4 av = *(const uint4*)(ap + ks * 32);
        const size_t o = (size_t)(2 * ks + ksub) * kOperandElems + lofs;
        const u32x4 v0 = __builtin_nontemporal_load((const u32x4*)(pb0 + o));
        const u32x4 v1 = __builtin_nontemporal_load((const u32x4*)(pb0 + o + 16 * 8));
        const u32x4 v2 = __builtin_nontemporal_load((const u32x4*)(pb1 + o));
        const u32x4 v3 = __builtin_nontemporal_load((const u32x4*)(pb1 + o + 16 * 8));
        const bf16x8_t a = as_bf16x8(av);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(v0), acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(v1), acc[1], 0, 0, 0);
        acc[2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(v2), acc[2], 0, 0, 0);
        acc[3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(v3), acc[3], 0, 0, 0);
      }
    } else {
      // k-steps in pairs (their loads issued together), an odd last one alone, into the
      // accumulators of the panel's two 16-column halves in k order
      int ks = 0;
      for (; ks + 1 < nks; ks += 2) {
        const uint4 av0 = *(const uint4*)(ap + ks * 32);
        const uint4 av1 = *(const uint4*)(ap + ks * 32 + 32);
        const size_t o0 = (size_t)(2 * ks + ksub) * kOperandElems + lofs;
        const size_t o1 = o0 + 2 * kOperandElems;
        const u32x4 v0 = __builtin_nontemporal_load((const u32x4*)(pb0 + o0));
        const u32x4 v1 = __builtin_nontemporal_load((const u32x4*)(pb0 + o0 + 16 * 8));
        const u32x4 w0 = __builtin_nontemporal_load((const u32x4*)(pb0 + o1));
        const u32x4 w1 = __builtin_nontemporal_load((const u32x4*)(pb0 + o1 + 16 * 8));
        __builtin_amdgcn_sched_barrier(0);  // all six loads in flight before the first MFMA
        const bf16x8_t a0 = as_bf16x8(av0), a1 = as_bf16x8(av1);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_bf16x8(v0), acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_bf16x8(v1), acc[1], 0, 0, 0);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, as_bf16x8(w0), acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, as_bf16x8(w1), acc[1], 0, 0, 0);
      }
      if (ks < nks) {
        const uint4 av0 = *(const uint4*)(ap + ks * 32);
        const size_t o0 = (size_t)(2 * ks + ksub) * kOperandElems + lofs;
        const u32x4 v0 = __builtin_nontemporal_load((const u32x4*)(pb0 + o0));
        const u32x4 v1 = __builtin_nontemporal_load((const u32x4*)(pb0 + o0 + 16 * 8));
        const bf16x8_t a0 = as_bf16x8(av0);
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_bf16x8(v0), acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_bf16x8(v1), acc[1], 0, 0, 0);
      }
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
        if constexpr (SAVE_GU) {  // g|u as the plain GEMM stores them (columns 64 g ..)
          uint16_t* o2 = gu + (size_t)(row_beg + r) * 2 * Nout + g * 64 + (lane & 15);
          o2[0] = to_bf16(acc[0][i]);
          o2[16] = to_bf16(acc[1][i]);
          o2[32] = to_bf16(acc[2][i]);
          o2[48] = to_bf16(acc[3][i]);
        }
      } else {
        const int c = g * 32 + (lane & 15);
        o[c] = to_bf16(acc[0][i]);
        o[c + 16] = to_bf16(acc[1][i]);
      }
    }
  }
}

}  // namespace

hipError_t launch_wgrad_bf16(const void* AT, const void* BT, const int32_t* poff, int E, int M,
                             int Ncols, int64_t npad, bool gu_split, float* out, float* out2,
                             hipStream_t s) {
  const dim3 grid(div_up(M, kPrefillBM), div_up(Ncols, 64 * kWaves), E);
  hipLaunchKernelGGL(wgrad_kernel, grid, dim3(kThreads), 0, s, (const uint16_t*)AT,
                     (const uint16_t*)BT, poff, M, Ncols, (int)npad, gu_split ? 1 : 0, out, out2);
  return hipGetLastError();
}

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

namespace {
template <bool GATHER, bool SAVE_GU>
void gate_up_bf16(const moe_problem& p, const void* xs, const int32_t* row_token,
                  const int32_t* offsets, const void* packed_gu, void* a, void* gu, bool decode,
                  hipStream_t s, int* claim) {
  if (decode) {
    const int nf32 = p.I / 32;
    hipLaunchKernelGGL((decode_kernel<true, GATHER, SAVE_GU>), dim3(div_up(nf32, 4), p.E),
                       dim3(256), 0, s, (const uint16_t*)xs, row_token, offsets,
                       (const uint16_t*)packed_gu, (uint16_t*)a, p.H, p.I, (uint16_t*)gu);
  } else {
    hipLaunchKernelGGL((prefill_kernel<true, GATHER, SAVE_GU>), dim3(persistent_grid()),
                       dim3(kThreads), 0, s, (const uint16_t*)xs, row_token, offsets, p.E,
                       (const uint16_t*)packed_gu, (uint16_t*)a, p.H, p.I, (uint16_t*)gu, claim);
  }
}
}  // namespace

hipError_t launch_gate_up_bf16(const moe_problem& p, const void* xs, const int32_t* row_token,
                               const int32_t* offsets, const void* packed_gu, void* a, void* gu,
                               bool decode, hipStream_t s, int* claim) {
  if (row_token && gu)
    gate_up_bf16<true, true>(p, xs, row_token, offsets, packed_gu, a, gu, decode, s, claim);
  else if (row_token)
    gate_up_bf16<true, false>(p, xs, row_token, offsets, packed_gu, a, nullptr, decode, s, claim);
  else if (gu)
    gate_up_bf16<false, true>(p, xs, nullptr, offsets, packed_gu, a, gu, decode, s, claim);
  else
    gate_up_bf16<false, false>(p, xs, nullptr, offsets, packed_gu, a, nullptr, decode, s, claim);
  return hipGetLastError();
}

// A plain grouped GEMM (the down projection's kernels) with any K and N: out[r] =
// A[r] B[e] (rows through row_token if not NULL), B packed like the down weights
// ([e][n32][k16] blocks), bf16 out.  The backward pass's data-gradient GEMMs.
hipError_t launch_gemm_bf16(int E, const void* A, const int32_t* row_token,
                            const int32_t* offsets, const void* packed_b, void* out, int K,
                            int Nout, bool decode, hipStream_t s) {
  const int nf32 = Nout / 32;
  if (decode) {
    if (row_token)
      hipLaunchKernelGGL((decode_kernel<false, true>), dim3(div_up(nf32, 4), E), dim3(256), 0,
                         s, (const uint16_t*)A, row_token, offsets, (const uint16_t*)packed_b,
                         (uint16_t*)out, K, Nout, nullptr);
    else
      hipLaunchKernelGGL((decode_kernel<false, false>), dim3(div_up(nf32, 4), E), dim3(256),
                         0, s, (const uint16_t*)A, nullptr, offsets, (const uint16_t*)packed_b,
                         (uint16_t*)out, K, Nout, nullptr);
  } else {
    if (row_token)
      hipLaunchKernelGGL((prefill_kernel<false, true>), dim3(persistent_grid()), dim3(kThreads),
                         0, s, (const uint16_t*)A, row_token, offsets, E,
                         (const uint16_t*)packed_b, (uint16_t*)out, K, Nout, nullptr, nullptr);
    else
      hipLaunchKernelGGL((prefill_kernel<false, false>), dim3(persistent_grid()),
                         dim3(kThreads), 0, s, (const uint16_t*)A, nullptr, offsets, E,
                         (const uint16_t*)packed_b, (uint16_t*)out, K, Nout, nullptr, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_down_bf16(const moe_problem& p, const void* a, const int32_t* offsets,
                            const void* packed_d, void* yp, bool decode, hipStream_t s,
                            int* claim) {
  if (decode) {
    const int nf32 = p.H / 32;
    hipLaunchKernelGGL((decode_kernel<false, false>), dim3(div_up(nf32, 4), p.E), dim3(256),
                       0, s, (const uint16_t*)a, nullptr, offsets, (const uint16_t*)packed_d,
                       (uint16_t*)yp, p.I, p.H, nullptr);
  } else {
    hipLaunchKernelGGL((prefill_kernel<false, false>), dim3(persistent_grid()), dim3(kThreads),
                       0, s, (const uint16_t*)a, nullptr, offsets, p.E,
                       (const uint16_t*)packed_d, (uint16_t*)yp, p.I, p.H, nullptr, claim);
  }
  return hipGetLastError();
}

}  // namespace moe
