// Plain grouped GEMM in bf16 on the gfx950 matrix cores (fp32 accumulation) over the expert
// prefix-sum layout, for problems with many rows per expert (the matrix cores, not the
// weight stream, bound them): out[r] = A[r] B[e] for the rows r of expert e -- the down
// projection yp = a W_down, and the backward pass's data-gradient GEMMs.
//
// LightLLM PR #1687 (PR body): the expert GEMMs run on the expert prefix-sum layout; the
// row count of every expert is data dependent and is read on the device from `offsets`.
//
// Tile: 256 rows x 256 columns (8 packed 32-column operand panels) per block of 8
// wavefronts (two per SIMD); wavefront (wm, wn) owns rows 128 wm .. + 128 and panels
// 2 wn, 2 wn + 1, as 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16.  Both operands go
// through LDS, copied straight from global memory (global_load_lds_dwordx4, no register
// staging):
//   the A rows in granules of 64 along K (256 rows x 128 bytes: whole cache lines), two
//     buffers, a granule's copies issued two stages before it is read;
//   the weights in stages of 32 along K (8 panels x 2 k-steps x one 1 KiB packed operand
//     block), a ring of five slots, copies four stages ahead.
// Per stage of 32 the L2 -> CU traffic is 32 KiB for 4.2 MFLOP (128 flop per byte, against
// 102 for the 128 x 512 tile of the other grouped GEMM kernel).  A tile accumulates its
// products in the same order as that kernel (k-steps of 16 in increasing K, the same
// instruction), so the two give the same bits.
//
// Scheduling (persistent, one block per CU): work item = (expert, N tile, M tile), in that
// order, so that the M tiles of an expert that read the same weight panel are adjacent in
// the item list and run at the same time; the item list is split into 8 contiguous
// ranges, one per XCD (block b runs on XCD b % 8), so those tiles meet in one XCD's L2.
// A block's copies form one continuous stream across its items: while it finishes an item
// the copies of the next item's first stages are already in flight, and the epilogue (the
// output tile through LDS in 16-byte row pieces) runs in the granule buffer just read.
//
// The copies are inline assembly: the compiler's wait-count pass, which cannot tell the
// ring slots apart, would otherwise wait for every copy in flight before each LDS read.
// Every wavefront issues the same copies per stage (see the stage barriers for the counts
// this implies); a wavefront waits for its own copies with vmcnt, then an s_barrier makes
// every wavefront's copies visible and frees the buffers read before it.
#include "bf16.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16), aligned(4)));

constexpr int kXcds = 8;
constexpr int kMaxExperts = 1024;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileRows = 256;
constexpr int kTilePanels = 8;       // 32-column operand panels per N tile
constexpr int kStageK = 32;          // K elements per stage (two k-steps of 16)
constexpr int kBSlots = 5;           // weight ring: copies run 4 stages ahead
constexpr int kBSlotBytes = 16384;   // 8 panels x 2 k-steps x 1 KiB
constexpr int kABufBytes = 32768;    // token rows of a granule: 256 rows x 64 K x 2 B
constexpr int kOperandElems = 512;   // one packed 32 x 16 operand block (1 KiB)

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// 16 bytes per lane from global memory into LDS: lane L's bytes land at LDS byte
// lds + 16 L (lds is wave-uniform; M0 holds it).
__device__ __forceinline__ void copy_to_lds(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// Stage barriers.  Per wavefront the copies go out in this order: at an even stage s the
// token rows of granule s / 2 + 1 (4 copies) then the weights of stage s + 4 (2 copies); at
// an odd stage the weights of stage s + 4 (2 copies).  So at the top of an even stage 2q the
// granule q (issued at stage 2q - 2, followed by 4 weight copies) has landed once at most 4
// operations are outstanding, and with it the older weights of stage 2q; at the top of an
// odd stage 2q + 1 its weights (issued at stage 2q - 3, followed by 14 copies) have landed
// once at most 14 are outstanding.  (Loads complete in order; anything issued later, such
// as an epilogue's stores, only makes the wait stricter.)  The s_barrier then makes every
// wavefront's copies visible, and (with lgkmcnt(0): this wavefront's LDS reads are done)
// frees the slots read in the previous stage.
__device__ __forceinline__ void barrier_even() {
  asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier_odd() {
  asm volatile("s_waitcnt vmcnt(14) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Token-row swizzle (granule rows of 128 bytes, 8 chunks of 16): row r's chunk c is stored
// at chunk position c ^ f(r), f(r) = ((r >> 1) ^ (r << 2)) & 7.  f takes 8 distinct values
// on any 8 consecutive rows and on the even (and the odd) rows of any 16, so a fragment read
// (32 rows x one chunk) is free of bank conflicts whether the LDS serves 8 or 16 lanes of
// 16-byte accesses per cycle.  f depends on r mod 16 only.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r << 2)) & 7; }

// Copy sources of one work item for this lane.  Token rows: wavefront w copies rows
// 32 w .. 32 w + 31 of the tile, 8 rows (one 1 KiB copy) at a time, lane L taking row
// 32 w + 8 q + L / 8 and its chunk (L % 8) ^ f(row); weights: wavefront w copies panel w.
struct SrcA {
  const uint16_t* r[4];
};
struct SrcB {
  const uint16_t* b;  // panel w of the N tile, k-step 0, lane L's 16 bytes
};

// What an item is: expert, N tile, M tile.
struct Item {
  int e, nt, mt;
};

struct Sched {
  const int* s_start;  // LDS: M tiles before expert e (exclusive scan), [E + 1]
  int E, ntn;
};

__device__ __forceinline__ Item item_of(const Sched& S, int it) {
  const int m = it / S.ntn;  // the item's M-tile index over all experts
  int lo = 0, hi = S.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (S.s_start[mid] <= m) lo = mid; else hi = mid;
  }
  const int e = lo;
  const int nmt = S.s_start[e + 1] - S.s_start[e];
  const int local = it - S.ntn * S.s_start[e];
  Item r;
  r.e = e;
  r.nt = local / nmt;
  r.mt = local - r.nt * nmt;
  return r;
}

template <bool GATHER>
__device__ __forceinline__ SrcA src_a_of(const Item& I, const uint16_t* A,
                                         const int32_t* __restrict__ row_token,
                                         const int32_t* __restrict__ offsets, int K, int wave,
                                         int lane) {
  const int row0 = offsets[I.e] + I.mt * kTileRows;
  const int rows = min(kTileRows, offsets[I.e + 1] - row0);
  const int j = lane >> 3;
  int t[4];
  if constexpr (GATHER) {
    // the wavefront's 32 token indices with uniform (scalar) loads: no vector-memory
    // operation that would have to be waited for behind the copies in flight (a whole
    // 32-row window in two 16-dword loads; a window that runs past the tile's rows takes
    // the tile's last row there)
    const int* rp = row_token + row0 + 32 * wave;
    t[0] = t[1] = t[2] = t[3] = 0;
    if (32 * wave + 32 <= rows) {
      const i32x16 w0 = *(const i32x16*)rp;
      const i32x16 w1 = *(const i32x16*)(rp + 16);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        t[0] = j == q ? w0[q] : t[0];
        t[1] = j == q ? w0[8 + q] : t[1];
        t[2] = j == q ? w1[q] : t[2];
        t[3] = j == q ? w1[8 + q] : t[3];
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int v = row_token[row0 + min(32 * wave + 8 * h + q, rows - 1)];
          t[h] = j == q ? v : t[h];
        }
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) t[h] = row0 + min(32 * wave + 8 * h + j, rows - 1);
  }
  SrcA s;
#pragma unroll
  for (int h = 0; h < 4; ++h)
    s.r[h] = A + (size_t)t[h] * K + (((lane & 7) ^ swz(8 * h + j)) * 8);
  return s;
}

__device__ __forceinline__ SrcB src_b_of(const Item& I, const uint16_t* Bp, int npan,
                                         size_t panel_elems, int wave, int lane) {
  const int pan = min(I.nt * kTilePanels + wave, npan - 1);
  SrcB s;
  s.b = Bp + ((size_t)I.e * npan + pan) * panel_elems + lane * 8;
  return s;
}

// The copy streams of a block: token-row granule `ga` of its ka-th item and weight stage
// `sb` of its kb-th item are the next to copy.  Past the block's last item each stream
// repeats its last copy (into a buffer nobody reads again), so that every wavefront issues
// the same copies per stage to the end.
struct Loader {
  SrcA a;
  SrcB b;
  int ka, ga, kb, sb;
  int abuf;  // A buffer of the next granule copy
  int bslot; // B slot of the next stage copy
};

template <bool GATHER>
struct Ctx {
  const Sched* S;
  const uint16_t* A;
  const int32_t* row_token;
  const int32_t* offsets;
  const uint16_t* Bp;
  int K, npan, nst, first, step, last;  // items first, first + step, ... <= last
  size_t panel_elems;
  uint32_t lds_a, lds_b;                // LDS byte offsets of the two rings
  int wave, lane;

  __device__ __forceinline__ void copy_a(Loader& L) {
    const uint32_t dst = lds_a + L.abuf * kABufBytes + wave * 4096;
    const size_t o = (size_t)L.ga * 2 * kStageK;
#pragma unroll
    for (int h = 0; h < 4; ++h) copy_to_lds(L.a.r[h] + o, dst + h * 1024);
    L.abuf ^= 1;
    if (++L.ga == nst / 2) {
      const int nit = first + (L.ka + 1) * step;
      if (nit <= last) {
        ++L.ka;
        L.ga = 0;
        L.a = src_a_of<GATHER>(item_of(*S, nit), A, row_token, offsets, K, wave, lane);
      } else {
        L.ga = nst / 2 - 1;
      }
    }
  }
  __device__ __forceinline__ void copy_b(Loader& L) {
    const uint32_t dst = lds_b + L.bslot * kBSlotBytes + wave * 2048;
    const size_t o = (size_t)L.sb * 2 * kOperandElems;
    copy_to_lds(L.b.b + o, dst);
    copy_to_lds(L.b.b + o + kOperandElems, dst + 1024);
    L.bslot = L.bslot == kBSlots - 1 ? 0 : L.bslot + 1;
    if (++L.sb == nst) {
      const int nit = first + (L.kb + 1) * step;
      if (nit <= last) {
        ++L.kb;
        L.sb = 0;
        L.b = src_b_of(item_of(*S, nit), Bp, npan, panel_elems, wave, lane);
      } else {
        L.sb = nst - 1;
      }
    }
  }
};

// MFMAs of one stage: A fragments of k-steps 2 p and 2 p + 1 of the granule in `abuf`
// (aoff[k]: this lane's offset for k-step k, row block 0), B fragments of the two k-steps
// in `bslot`; wavefront rows 32 m + .. for m < NB.
template <int NB, class Mid>
__device__ __forceinline__ void compute_stage(f32x16_t (&acc)[4][2], const char* abuf, int ao0,
                                              int ao1, const char* bslot, int boff, Mid mid) {
  if constexpr (NB == 0) {
    mid();
  } else {
    bf16x8_t a0[NB], a1[NB], b0[2], b1[2];
#pragma unroll
    for (int m = 0; m < NB; ++m)
      a0[m] = __builtin_bit_cast(bf16x8_t, *(const u32x4*)(abuf + ao0 + m * 4096));
#pragma unroll
    for (int h = 0; h < 2; ++h)
      b0[h] = __builtin_bit_cast(bf16x8_t, *(const u32x4*)(bslot + boff + h * 2048));
#pragma unroll
    for (int m = 0; m < NB; ++m)
      a1[m] = __builtin_bit_cast(bf16x8_t, *(const u32x4*)(abuf + ao1 + m * 4096));
#pragma unroll
    for (int h = 0; h < 2; ++h)
      b1[h] = __builtin_bit_cast(bf16x8_t, *(const u32x4*)(bslot + boff + h * 2048 + 1024));
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[m], b0[0], acc[m][0], 0, 0, 0);
      acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[m], b0[1], acc[m][1], 0, 0, 0);
    }
    // the stage's copies go out behind the first k-step's MFMAs
    mid();
#pragma unroll
    for (int m = 0; m < NB; ++m) {
      acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[m], b1[0], acc[m][0], 0, 0, 0);
      acc[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[m], b1[1], acc[m][1], 0, 0, 0);
    }
  }
}

// Output of one item for this wavefront (32 x 64 blocks through its own 4 KiB of LDS scratch
// within the granule buffer just read, stored as 16-byte row pieces).
//   out : the wavefront's first output element (row 128 wm of the tile, its first column)
// 32x32 accumulator layout: element i of lane l is row 8 (i / 4) + 4 (l / 32) + i % 4,
// column l % 32.
template <int NB>
__device__ __forceinline__ void epilogue(const f32x16_t (&acc)[4][2], char* scratch, int lane,
                                         int rows, bool act, uint16_t* out, int Nout) {
  uint16_t* const lds16 = reinterpret_cast<uint16_t*>(scratch);
  const int wofs = (lane >> 5) * 4 * 64 + (lane & 31);
  const int qrow = lane >> 3, qcol = (lane & 7) * 8;
#pragma unroll
  for (int m = 0; m < NB; ++m) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint16_t* srow = lds16 + wofs + ((i >> 2) * 8 + (i & 3)) * 64;
      srow[0] = to_bf16(acc[m][0][i]);
      srow[32] = to_bf16(acc[m][1][i]);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int q0 = 0; q0 < 256; q0 += 64) {
      const int rr = qrow + q0 / 8;
      const int r = m * 32 + rr;
      const u32x4 v = *(const u32x4*)(lds16 + rr * 64 + qcol);
      if (act && r < rows) *(u32x4*)(out + (size_t)r * Nout + qcol) = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// Where the stream is in LDS: the A buffer of the granule being read, the B slot of the
// stage being read.
struct Cursor {
  int abuf, bslot;
};

// One item: its stages in pairs (an even stage starts a granule), then its epilogue.
template <int NB, bool GATHER>
__device__ __forceinline__ void run_item(Ctx<GATHER>& C, Loader& L, Cursor& U, char* lds_a,
                                         char* lds_b, const int (&aoff)[4], int boff, int rows,
                                         bool act, uint16_t* out, int Nout) {
  f32x16_t acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m][0] = acc[m][1] = f32x16_t{};
  for (int ls = 0; ls < C.nst; ls += 2) {
    const char* abuf = lds_a + U.abuf * kABufBytes;
    barrier_even();
    compute_stage<NB>(acc, abuf, aoff[0], aoff[1], lds_b + U.bslot * kBSlotBytes, boff, [&] {
      C.copy_a(L);
      C.copy_b(L);
    });
    U.bslot = U.bslot == kBSlots - 1 ? 0 : U.bslot + 1;
    barrier_odd();
    compute_stage<NB>(acc, abuf, aoff[2], aoff[3], lds_b + U.bslot * kBSlotBytes, boff,
                      [&] { C.copy_b(L); });
    U.bslot = U.bslot == kBSlots - 1 ? 0 : U.bslot + 1;
    U.abuf ^= 1;
  }
  // every wavefront is done reading the last granule's buffer: it becomes epilogue scratch
  lds_barrier();
  char* scratch = lds_a + (U.abuf ^ 1) * kABufBytes + C.wave * 4096;
  epilogue<NB>(acc, scratch, C.lane, rows, act, out, Nout);
}

// Bp: packed like the down weights ([e][n32][k16] blocks of 1 KiB), Nout output columns
// (a multiple of 64), K % 64 == 0.  GATHER: row r of the layout is A[row_token[r]] (token
// rows) instead of A[r].
template <bool GATHER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_kernel(const uint16_t* __restrict__ A, const int32_t* __restrict__ row_token,
                    const int32_t* __restrict__ offsets, int E, const uint16_t* __restrict__ Bp,
                    uint16_t* __restrict__ out, int K, int Nout) {
  __shared__ __attribute__((aligned(1024))) char lds_a[2 * kABufBytes];
  __shared__ __attribute__((aligned(1024))) char lds_b[kBSlots * kBSlotBytes];
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_wsum[kWaves];

  const int tid = threadIdx.x;
  // wave-uniform for the compiler too (scalar loads of row_token, copy addresses in M0)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  // ---- per-expert M-tile starts (exclusive scan of ceil(count / 256))
  {
    const int per = div_up(E, kThreads);
    const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
    int sum = 0;
    for (int e = e0; e < e1; ++e) sum += div_up(offsets[e + 1] - offsets[e], kTileRows);
    int inc = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(inc, d, 64);
      if (lane >= d) inc += u;
    }
    if (lane == 63) s_wsum[wave] = inc;
    __syncthreads();
    int base = inc - sum;
    for (int w = 0; w < wave; ++w) base += s_wsum[w];
    for (int e = e0; e < e1; ++e) {
      s_start[e] = base;
      base += div_up(offsets[e + 1] - offsets[e], kTileRows);
    }
    if (tid == kThreads - 1) s_start[E] = base;
    __syncthreads();
  }
  const int npan = Nout / 32;  // operand panels per expert
  const int ntn = div_up(npan, kTilePanels);
  Sched S{s_start, E, ntn};
  const int64_t total = (int64_t)s_start[E] * ntn;
  const int xcd = blockIdx.x % kXcds;
  const int slot = blockIdx.x / kXcds;
  const int nslots = gridDim.x / kXcds;
  const int lo = (int)(total * xcd / kXcds);
  const int hi = (int)(total * (xcd + 1) / kXcds);
  if (lo + slot >= hi) return;  // block-uniform: no work (no copy was issued)

  Ctx<GATHER> C;
  C.S = &S;
  C.A = A;
  C.row_token = row_token;
  C.offsets = offsets;
  C.Bp = Bp;
  C.K = K;
  C.npan = npan;
  C.nst = K / kStageK;  // even: K % 64 == 0
  C.first = lo + slot;
  C.step = nslots;
  C.last = hi - 1;
  C.panel_elems = (size_t)(K / 16) * kOperandElems;
  C.lds_a = lds_offset(lds_a);
  C.lds_b = lds_offset(lds_b);
  C.wave = wave;
  C.lane = lane;

  // fragment offsets of this lane: A (bytes within a granule buffer) per k-step, B (within
  // a weight slot)
  const int wm = wave >> 2, wn = wave & 3;
  const int fr = lane & 31;
  int aoff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    aoff[kk] = (128 * wm + fr) * 128 + (((2 * kk + (lane >> 5)) ^ swz(fr)) << 4);
  const int boff = (2 * wn) * 2048 + lane * 16;

  // the copy streams' start, in their steady-state order (weights of stages 0 and 1, token
  // rows of granule 0, weights of stages 2 and 3)
  Loader L;
  {
    const Item I0 = item_of(S, C.first);
    L.a = src_a_of<GATHER>(I0, A, row_token, offsets, K, wave, lane);
    L.b = src_b_of(I0, Bp, npan, C.panel_elems, wave, lane);
  }
  L.ka = L.ga = L.kb = L.sb = 0;
  L.abuf = L.bslot = 0;
  C.copy_b(L);
  C.copy_b(L);
  C.copy_a(L);
  C.copy_b(L);
  C.copy_b(L);
  Cursor U{0, 0};

  for (int it = C.first; it <= C.last; it += C.step) {
    const Item I = item_of(S, it);
    const int row0 = offsets[I.e] + I.mt * kTileRows;
    const int rows = min(kTileRows, offsets[I.e + 1] - row0) - 128 * wm;  // this wavefront's
    const int nb = rows <= 0 ? 0 : min(4, div_up(rows, 32));
    const int nf = I.nt * kTilePanels + 2 * wn;  // the wavefront's 64 output columns
    const bool act = nf < npan;
    uint16_t* const o = out + (size_t)(row0 + 128 * wm) * Nout + nf * 32;
    switch (nb) {
      case 4:
        run_item<4, GATHER>(C, L, U, lds_a, lds_b, aoff, boff, rows, act, o, Nout);
        break;
      case 3:
        run_item<3, GATHER>(C, L, U, lds_a, lds_b, aoff, boff, rows, act, o, Nout);
        break;
      case 2:
        run_item<2, GATHER>(C, L, U, lds_a, lds_b, aoff, boff, rows, act, o, Nout);
        break;
      case 1:
        run_item<1, GATHER>(C, L, U, lds_a, lds_b, aoff, boff, rows, act, o, Nout);
        break;
      default:
        run_item<0, GATHER>(C, L, U, lds_a, lds_b, aoff, boff, rows, act, o, Nout);
        break;
    }
  }
  // the copies past the last item must land before the block's LDS goes away
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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

hipError_t launch_grouped_bf16(int E, const void* A, const int32_t* row_token,
                               const int32_t* offsets, const void* packed_b, void* out, int K,
                               int Nout, hipStream_t s) {
  const dim3 grid(persistent_grid()), block(kThreads);
  if (row_token)
    hipLaunchKernelGGL((grouped_kernel<true>), grid, block, 0, s,
                       (const uint16_t*)A, row_token, offsets, E, (const uint16_t*)packed_b,
                       (uint16_t*)out, K, Nout);
  else
    hipLaunchKernelGGL((grouped_kernel<false>), grid, block, 0, s,
                       (const uint16_t*)A, nullptr, offsets, E, (const uint16_t*)packed_b,
                       (uint16_t*)out, K, Nout);
  return hipGetLastError();
}

}  // namespace moe
