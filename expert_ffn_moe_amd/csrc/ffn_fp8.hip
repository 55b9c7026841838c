// Grouped SwiGLU expert FFN with FP8 operands on the gfx950 scaled matrix cores.
//
// LightLLM PR #1687 (PR body): the expert GEMMs run in FP8 with UE8M0 scales on the
// prefix-sum layout, and the SwiGLU output is quantised before the down projection
// (`silu_and_mul_psum_post_quant`).  With x^, W^, a^ the dequantised operands
// (E4M3 codes times their block's power-of-two scale, blocks of 32 along K):
//   gate/up: a[r]  = quant(silu(x^[r] Wg^[e]) * (x^[r] Wu^[e]))   (codes + scales)
//   down   : yp[r] = a^[r] Wd^[e]                                   (bf16)
// One instruction, v_mfma_scale_f32_32x32x64_f8f6f4, multiplies a 32x64 by a 64x32 block
// of E4M3 codes and applies one E8M0 scale per row (column) and 32-element K block.
//
// The kernel is the bf16 prefill kernel's schedule with FP8 bytes: persistent, XCD-aware,
// 8 wavefronts, 128-row M tiles, wavefront tile 128 rows x 2 operand columns.  A stage of
// the K loop is one 128-byte line of every row (128 elements, two k-steps of 64): the
// activation codes go through LDS with the same swizzled layout, their scale bytes (4 per
// row and stage) through a small LDS array next to it, and the weight operands (2 KiB
// blocks, 32 bytes per lane) stream into a one-stage register ring.  Weight scale bytes
// come as one word per lane per 4 k-steps.  Operand layout of the instruction (checked on
// the device): lane l, half h = l / 32, holds row (column) l % 32 at k = 16h .. 16h + 15
// in bytes 0..15 and k = 32 + 16h .. in bytes 16..31; its scale byte is that of K block h.
#include <algorithm>

#include "bf16.h"
#include "fp8.h"
#include "moe_internal.h"
#include "wave.h"

namespace moe {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;
constexpr int kMaxExperts = 1024;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 128;            // rows per M tile
constexpr int kBlockBytes = 2048;   // one packed 32 x 64 operand block

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

__device__ __forceinline__ i32x8 join(const u32x4& lo, const u32x4& hi) {
  i32x8 r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

__device__ __forceinline__ i32x8 load_operand(const uint8_t* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  return join(q[0], q[1]);
}

// Maximum over the 32 lanes of each half wavefront.
__device__ __forceinline__ uint32_t half_wave_max(uint32_t v) {
  v = max(v, dpp_u32<kDppQuadXor1>(v));
  v = max(v, dpp_u32<kDppQuadXor2>(v));
  v = max(v, dpp_u32<kDppRowHalfMirror>(v));
  v = max(v, dpp_u32<kDppRowMirror>(v));
  v = max(v, (uint32_t)__shfl_xor((int)v, 16, 64));
  return v;
}

struct Tile8 {
  const uint8_t* A;      // activation codes of tile row 0 (with a gather: the token rows)
  const uint8_t* As;     // activation scales (same rows, row stride K / 32)
  const int32_t* rtok;   // gather: row_token + row0
  const uint8_t* b0;     // this wavefront's operand panels (lane offset applied)
  const uint8_t* b1;
  const uint32_t* bs0;   // their scale words (lane offset applied)
  const uint32_t* bs1;
  uint8_t* out;          // GATE_UP: a codes / DOWN: yp (bf16), at tile row 0, column col0
  uint8_t* outs;         // GATE_UP: a scales at tile row 0
  int K, Nout, rows, wave, lane, act, col0;
  int fb[2][2];          // LDS index of the lane's two 16-byte pieces per k-step (m = 0)
};

// Activation stage layout: 128 rows x 128 bytes, 16-byte chunk c of row r at chunk
// c ^ f(r), f(r) = ((r >> 1) ^ (r << 2)) & 7: conflict-free 8-row stores and 32-row reads.
__device__ __forceinline__ int a_slot(int r, int c) {
  return r * 8 + (c ^ (((r >> 1) ^ (r << 2)) & 7));
}

template <int NM, int BUF, int KK>
__device__ __forceinline__ void kstep(f32x16_t (&acc)[NM][2], i32x8 (&bring)[2][2],
                                      const u32x4 (*lds)[1024], const uint32_t (&asc)[NM],
                                      uint32_t bsc0, uint32_t bsc1, const Tile8& t,
                                      int j_next) {
  const u32x4* base = &lds[BUF][0];
  const int ash = 8 * (2 * KK + (t.lane >> 5));  // A: this lane's K block of the stage
  constexpr int bsh = 8 * (2 * BUF + KK);        // B: k-step within the group of 4
  const int sb0 = (int)((bsc0 >> bsh) & 0xFFu), sb1 = (int)((bsc1 >> bsh) & 0xFFu);
  // A fragments are read from LDS one 32-row block ahead of their MFMAs
  i32x8 a = join(base[t.fb[KK][0]], base[t.fb[KK][1]]);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    i32x8 an = a;
    if (m + 1 < NM)
      an = join(base[t.fb[KK][0] + 256 * (m + 1)], base[t.fb[KK][1] + 256 * (m + 1)]);
    const int sa = (int)((asc[m] >> ash) & 0xFFu);
    acc[m][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bring[KK][0], acc[m][0], 0,
                                                                0, 0, sa, 0, sb0);
    acc[m][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bring[KK][1], acc[m][1], 0,
                                                                0, 0, sa, 0, sb1);
    __builtin_amdgcn_sched_barrier(0);  // keeps at most two fragments in registers
    a = an;
  }
  const size_t o = (size_t)j_next * kBlockBytes;
  bring[KK][0] = load_operand(t.b0 + o);
  bring[KK][1] = load_operand(t.b1 + o);
  __builtin_amdgcn_sched_barrier(0);
}

// One stage (128 elements of K) from LDS buffer BUF; activation codes and scales for stage
// s + 2 are loaded into register set BUF, stage s + 1 (set 1 - BUF) is stored to LDS.
template <int NM, int BUF>
__device__ __forceinline__ void kstage(f32x16_t (&acc)[NM][2], i32x8 (&bring)[2][2],
                                       u32x4 (&aset)[2][2], uint32_t (&ascr)[2],
                                       u32x4 (*lds)[1024], uint32_t (*lds_s)[kThreads],
                                       const uint8_t* const (&ag)[2], const int (&lslot)[2],
                                       const uint8_t* asrc, uint32_t bsc0, uint32_t bsc1,
                                       const Tile8& t, int tid, int s, int nst) {
  const int sl = min(s + 2, nst - 1);
  aset[BUF][0] = *(const u32x4*)(ag[0] + (size_t)sl * 128);
  aset[BUF][1] = *(const u32x4*)(ag[1] + (size_t)sl * 128);
  ascr[BUF] = *(const uint32_t*)(asrc + 4 * sl);
  __builtin_amdgcn_sched_barrier(0);
  uint32_t asc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) asc[m] = lds_s[BUF][32 * m + (t.lane & 31)];
  const int jn = 2 * (s + 1), jmax = 2 * nst - 1;
  kstep<NM, BUF, 0>(acc, bring, lds, asc, bsc0, bsc1, t, min(jn, jmax));
  kstep<NM, BUF, 1>(acc, bring, lds, asc, bsc0, bsc1, t, min(jn + 1, jmax));
  lds[1 - BUF][lslot[0]] = aset[1 - BUF][0];
  lds[1 - BUF][lslot[1]] = aset[1 - BUF][1];
  lds_s[1 - BUF][tid] = ascr[1 - BUF];
  __syncthreads();
}

// One work item: NM 32-row blocks (NM = 4, or 2 / 1 for a tile with at most 64 / 32 rows) x this
// wavefront's two operand columns.
template <bool GATE_UP, bool GATHER, int NM>
__device__ __forceinline__ void tile8(const Tile8& t, u32x4 (*lds)[1024], uint32_t (*lds_s)[kThreads],
                                      int tid) {
  const int nst = t.K / 128;
  const int lane = t.lane, wave = t.wave;
  // activation loader: load p of wavefront w covers rows 64p + 8w .. + 7, lane L taking
  // 16-byte chunk L % 8 of row L / 8 (whole 128-byte lines); thread tid loads the stage's
  // 4 scale bytes of row tid % 128 (threads >= 128 load copies, so the loop has no branch)
  const uint8_t* ag[2];
  int lslot[2];
  const int lr = wave * 8 + (lane >> 3), lc = lane & 7;
  const int lbase = a_slot(lr, lc);
  const size_t sstride = (size_t)t.K / kQBlock;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int r = min(p * 64 + lr, t.rows - 1);
    const size_t src = GATHER ? (size_t)t.rtok[r] : (size_t)r;
    ag[p] = t.A + src * t.K + lc * 16;
    lslot[p] = lbase + 512 * p;
  }
  const uint8_t* asrc;
  {
    const int r = min(tid & (kBM - 1), t.rows - 1);
    const size_t src = GATHER ? (size_t)t.rtok[r] : (size_t)r;
    asrc = t.As + src * sstride;
  }
  f32x16_t acc[NM][2];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m][0] = acc[m][1] = f32x16_t{};
  u32x4 aset[2][2];
  uint32_t ascr[2] = {0u, 0u};
  i32x8 bring[2][2];
  const int s1 = min(1, nst - 1);
  aset[0][0] = *(const u32x4*)(ag[0]);
  aset[0][1] = *(const u32x4*)(ag[1]);
  aset[1][0] = *(const u32x4*)(ag[0] + (size_t)s1 * 128);
  aset[1][1] = *(const u32x4*)(ag[1] + (size_t)s1 * 128);
  ascr[0] = *(const uint32_t*)(asrc);
  ascr[1] = *(const uint32_t*)(asrc + 4 * s1);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const size_t o = (size_t)min(q, 2 * nst - 1) * kBlockBytes;
    bring[q][0] = load_operand(t.b0 + o);
    bring[q][1] = load_operand(t.b1 + o);
  }
  uint32_t bsc0 = t.bs0[0], bsc1 = t.bs1[0];
  lds[0][lslot[0]] = aset[0][0];
  lds[0][lslot[1]] = aset[0][1];
  lds_s[0][tid] = ascr[0];
  __syncthreads();
  // stages in pairs (a scale word covers 4 k-steps = 2 stages), an odd last stage after
  const int ngroups = div_up(nst, 2);
  for (int s0 = 0; s0 + 1 < nst; s0 += 2) {
    const int gn = min(s0 / 2 + 1, ngroups - 1);
    const uint32_t nb0 = t.bs0[64 * gn], nb1 = t.bs1[64 * gn];
    kstage<NM, 0>(acc, bring, aset, ascr, lds, lds_s, ag, lslot, asrc, bsc0, bsc1, t, tid, s0, nst);
    kstage<NM, 1>(acc, bring, aset, ascr, lds, lds_s, ag, lslot, asrc, bsc0, bsc1, t, tid, s0 + 1,
                  nst);
    bsc0 = nb0;
    bsc1 = nb1;
  }
  if (nst & 1)
    kstage<NM, 0>(acc, bring, aset, ascr, lds, lds_s, ag, lslot, asrc, bsc0, bsc1, t, tid, nst - 1,
                  nst);

  // Epilogue through LDS, per 32-row fragment (accumulator element i of lane l: row
  // 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32).
  const int h = lane >> 5, col = lane & 31;
  if constexpr (GATE_UP) {
    // a = silu(gate) * up, quantised per row and 32-column block (this wavefront's 32
    // columns are one block): amax over the 32 lanes holding the row, scale, E4M3 codes.
    uint8_t* l8 = reinterpret_cast<uint8_t*>(&lds[0][0]) + wave * 2048;  // [32][32] + [32]
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m * 32 < t.rows) {  // block-uniform
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 8 * (i >> 2) + 4 * h + (i & 3);
          const float v = silu_mul(acc[m][0][i], acc[m][1][i]);
          const uint32_t amax = half_wave_max(__float_as_uint(v) & 0x7FFFFFFFu);
          const int e = ue8m0_exp(__uint_as_float(amax));
          const int q = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v, -e), 0.0f, 0, false);
          l8[row * 32 + col] = (uint8_t)(q & 0xFF);
          if (col == 0) l8[1024 + row] = (uint8_t)(e + 127);
        }
        __syncthreads();
        const int rr = lane >> 1, half = lane & 1;
        const int r = m * 32 + rr;
        if (t.act && r < t.rows)
          *(u32x4*)(t.out + (size_t)r * t.Nout + t.col0 + 16 * half) =
              *(const u32x4*)(l8 + rr * 32 + 16 * half);
        if (t.act && lane < 32 && m * 32 + lane < t.rows)
          t.outs[(size_t)(m * 32 + lane) * (t.Nout / kQBlock) + t.col0 / kQBlock] = l8[1024 + lane];
        __syncthreads();
      }
    }
  } else {
    // bf16 yp: each wavefront writes its 32 x 64 block row-major into LDS, then stores
    // whole 16-byte row pieces
    uint16_t* l16 = reinterpret_cast<uint16_t*>(&lds[0][0]) + wave * 2048;
    const int wofs = h * 4 * 64 + col;
    const int qrow = lane / 8, qcol = (lane % 8) * 8;
    uint16_t* out = reinterpret_cast<uint16_t*>(t.out);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m * 32 < t.rows) {  // block-uniform
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          uint16_t* srow = l16 + wofs + ((i >> 2) * 8 + (i & 3)) * 64;
          srow[0] = to_bf16(acc[m][0][i]);
          srow[32] = to_bf16(acc[m][1][i]);
        }
        __syncthreads();
#pragma unroll
        for (int q0 = 0; q0 < 256; q0 += 64) {
          const int rr = qrow + q0 / 8;
          const int r = m * 32 + rr;
          if (t.act && r < t.rows)
            *(u32x4*)(out + (size_t)r * t.Nout + t.col0 + qcol) =
                *(const u32x4*)(l16 + rr * 64 + qcol);
        }
        __syncthreads();
      }
    }
  }
}

// Persistent grouped GEMM (scheduling as in the bf16 prefill kernel).
//   GATE_UP: A = x codes/scales (token rows with GATHER), out = a codes, outs = a scales
//   DOWN   : A = a codes/scales, out = yp (bf16)
template <bool GATE_UP, bool GATHER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fp8_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                const int32_t* __restrict__ row_token, const int32_t* __restrict__ offsets,
                int E, const uint8_t* __restrict__ Bq, const uint32_t* __restrict__ Bs,
                uint8_t* __restrict__ out, uint8_t* __restrict__ outs, int K, int Nout) {
  __shared__ u32x4 lds_a[2][1024];
  __shared__ uint32_t lds_s[2][kThreads];  // entries >= kBM: unused copies (no branch)
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_wsum[kWaves];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  {
    const int per = div_up(E, kThreads);
    const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
    int sum = 0;
    for (int e = e0; e < e1; ++e) sum += div_up(offsets[e + 1] - offsets[e], kBM);
    const int inc = wave_inclusive_scan(sum);
    if (lane == 63) s_wsum[wave] = inc;
    __syncthreads();
    int base = inc - sum;
    for (int w = 0; w < wave; ++w) base += s_wsum[w];
    for (int e = e0; e < e1; ++e) {
      s_start[e] = base;
      base += div_up(offsets[e + 1] - offsets[e], kBM);
    }
    if (tid == kThreads - 1) s_start[E] = base;
    __syncthreads();
  }
  const int total_mt = s_start[E];
  const int nks = K / 64;
  const int nf32 = Nout / 32;
  const int ntn = GATE_UP ? div_up(nf32, kWaves) : div_up(nf32, 2 * kWaves);
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int mt_lo = (int)((int64_t)total_mt * xcd / kXcds);
  const int mt_hi = (int)((int64_t)total_mt * (xcd + 1) / kXcds);
  const int items = (mt_hi - mt_lo) * ntn;
  const size_t panel = (size_t)nks * kBlockBytes;
  const size_t spanel = (size_t)div_up(nks, 4) * 64;  // scale words per panel

  for (int item = slot; item < items; item += nslots) {
    // expert by expert, N group major and M tile minor, as in the bf16 prefill kernel: the
    // expert is that of tile mt_lo + item / ntn
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
    const int row0 = offsets[e] + (mt - s_start[e]) * kBM;
    Tile8 t;
    t.rows = min(kBM, offsets[e + 1] - row0);
    t.K = K;
    t.Nout = Nout;
    t.wave = wave;
    int lane_v = lane;
    __asm__ volatile("" : "+v"(lane_v));  // keep lane-derived addresses per item
    t.lane = lane_v;
    size_t p0;  // first panel index of this wavefront
    if (GATE_UP) {
      int af = nt * kWaves + wave;
      t.act = af < nf32;
      af = min(af, nf32 - 1);
      p0 = (size_t)(e * nf32 + af) * 2;
      t.col0 = af * 32;
    } else {
      int nf = (nt * kWaves + wave) * 2;
      t.act = nf < nf32;
      nf = min(nf, nf32 - 2);
      p0 = (size_t)(e * nf32 + nf);
      t.col0 = nf * 32;
    }
    t.b0 = Bq + p0 * panel + lane_v * 32;
    t.b1 = t.b0 + panel;
    t.bs0 = Bs + p0 * spanel + lane_v;
    t.bs1 = t.bs0 + spanel;
    t.A = GATHER ? A : A + (size_t)row0 * K;
    t.As = GATHER ? As : As + (size_t)row0 * (K / kQBlock);
    t.rtok = GATHER ? row_token + row0 : nullptr;
    t.out = GATE_UP ? out + (size_t)row0 * Nout : out + (size_t)row0 * Nout * 2;
    t.outs = GATE_UP ? outs + (size_t)row0 * (Nout / kQBlock) : nullptr;
    const int lrow = lane_v & 31, hh = lane_v >> 5;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      t.fb[kk][0] = a_slot(lrow, 4 * kk + hh);
      t.fb[kk][1] = a_slot(lrow, 4 * kk + 2 + hh);
    }
    if (t.rows > 64)  // block-uniform
      tile8<GATE_UP, GATHER, 4>(t, lds_a, lds_s, tid);
    else if (t.rows > 32)
      tile8<GATE_UP, GATHER, 2>(t, lds_a, lds_s, tid);
    else
      tile8<GATE_UP, GATHER, 1>(t, lds_a, lds_s, tid);
  }
}

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

hipError_t launch_gate_up_fp8(const moe_problem& p, const uint8_t* xq, const uint8_t* xs,
                              const int32_t* row_token, const int32_t* offsets,
                              const void* packed_gu, uint8_t* aq, uint8_t* as, hipStream_t s) {
  const uint8_t* bq = (const uint8_t*)packed_gu;
  const uint32_t* bs = (const uint32_t*)(bq + align256(fp8_packed_code_bytes(p.E, p.H, p.I, 2)));
  if (row_token)
    hipLaunchKernelGGL((fp8_kernel<true, true>), dim3(persistent_grid()), dim3(kThreads), 0, s,
                       xq, xs, row_token, offsets, p.E, bq, bs, aq, as, p.H, p.I);
  else
    hipLaunchKernelGGL((fp8_kernel<true, false>), dim3(persistent_grid()), dim3(kThreads), 0, s,
                       xq, xs, nullptr, offsets, p.E, bq, bs, aq, as, p.H, p.I);
  return hipGetLastError();
}

hipError_t launch_down_fp8(const moe_problem& p, const uint8_t* aq, const uint8_t* as,
                           const int32_t* offsets, const void* packed_d, void* yp,
                           hipStream_t s) {
  const uint8_t* bq = (const uint8_t*)packed_d;
  const uint32_t* bs = (const uint32_t*)(bq + align256(fp8_packed_code_bytes(p.E, p.I, p.H, 1)));
  hipLaunchKernelGGL((fp8_kernel<false, false>), dim3(persistent_grid()), dim3(kThreads), 0, s,
                     aq, as, nullptr, offsets, p.E, bq, bs, (uint8_t*)yp, nullptr, p.I, p.H);
  return hipGetLastError();
}

}  // namespace moe
