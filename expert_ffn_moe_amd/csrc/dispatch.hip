// Local dispatch: per-expert capacity, expert histogram + prefix scan, stable scatter and
// row gather.
//
// Layout (LightLLM PR #1687, PR body: the grouped GEMM runs on the expert prefix-sum
// layout): rows of expert e occupy [offsets[e], offsets[e+1]) with offsets the exclusive
// scan of the per-expert counts; inside a segment rows ascend in token index.  On one GPU
// this permutation stands in for the dispatch all-to-all (research-vault WideEP card).
//
// Capacity (docs.axolotl.ai expert-parallel args, `expert_parallel_token_capacity`): an
// expert with more than C candidate assignments keeps the C with the largest
// (weight, -token) key; the rest are dropped.
//
// Determinism: every count comes from popcounts of per-chunk bitmaps (one bit per token
// of a 64-token chunk), every rank from a popcount of the bits below the token, every
// sum from a fixed-order scan.  LDS atomics only set bits or count into a histogram,
// whose results do not depend on their order.
#include "moe_internal.h"
#include "wave.h"

namespace moe {
namespace {

// Whether a routed slot's expert id may index the layout.  Ids are a documented device-side
// precondition ([0, E), distinct within a token); a build with MOE_DEBUG_CHECKS checks them
// (launch_check_ids) and treats a slot whose id lies outside [0, E) as dropped, so that an
// invalid id is reported instead of indexing out of bounds.  (A repeated id stays in bounds:
// its slots share one row.)
__device__ __forceinline__ bool id_usable(int e, int E) {
#ifdef MOE_DEBUG_CHECKS
  return (unsigned)e < (unsigned)E;
#else
  (void)e;
  (void)E;
  return true;
#endif
}

// Chunks (wavefronts) per block of the histogram and scatter launches: one, so that the
// scattered row stores of a layout spread over as many CUs as it has chunks.
constexpr int kLayoutWaves = 1;

// Slots are read in batches of kBatch (all loads issued before the first use: the LDS
// atomics that consume them would otherwise wait for each load in turn).
constexpr int kBatch = 8;

// The expert id of slot s if the slot exists and is kept, else -1 (the id and the keep flag
// are loaded independently, so that neither waits for the other).
template <bool HAS_KEEP>
__device__ __forceinline__ int load_slot(const int32_t* __restrict__ ids,
                                         const uint8_t* __restrict__ keep, size_t s, bool exists) {
  if (!exists) return -1;
  const int e = ids[s];
  return (!HAS_KEEP || keep[s]) ? e : -1;
}

// Builds, for the chunk of 64 tokens handled by this wavefront, the bitmap
// bm[e] = {lanes whose token has a (kept) slot routed to e}.  Call from all threads of
// the block (contains barriers).
template <bool HAS_KEEP>
__device__ __forceinline__ void build_chunk_bitmap(uint64_t* bm, const int32_t* __restrict__ ids,
                                                   const uint8_t* __restrict__ keep, int T,
                                                   int E, int k, int c, int nchunks) {
  const int lane = threadIdx.x & 63;
  for (int e = lane; e < E; e += 64) bm[e] = 0;
  __syncthreads();
  const int t = c * kChunk + lane;
  if (c < nchunks && t < T) {
    for (int j0 = 0; j0 < k; j0 += kBatch) {
      int ev[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const size_t s = (size_t)t * k + j0 + j;
        ev[j] = load_slot<HAS_KEEP>(ids, keep, s, j0 + j < k);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (ev[j] != -1 && id_usable(ev[j], E))
          atomicOr((unsigned long long*)&bm[ev[j]], 1ull << lane);
    }
  }
  __syncthreads();
}

template <bool HAS_KEEP>
__global__ __launch_bounds__(64 * kLayoutWaves) void chunk_hist_kernel(const int32_t* __restrict__ ids,
                                                         const uint8_t* __restrict__ keep, int T,
                                                         int E, int k, int nchunks,
                                                         int32_t* __restrict__ chunk_hist) {
  extern __shared__ uint64_t smem_bm[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * kLayoutWaves + wave;
  uint64_t* bm = smem_bm + (size_t)wave * E;
  build_chunk_bitmap<HAS_KEEP>(bm, ids, keep, T, E, k, c, nchunks);
  if (c < nchunks)
    for (int e = lane; e < E; e += 64) chunk_hist[(size_t)c * E + e] = __popcll(bm[e]);
}

// Column scan: 64 experts per block (one per lane), 16 wavefronts split the chunks.
__global__ __launch_bounds__(1024) void scan_cols_kernel(const int32_t* __restrict__ chunk_hist,
                                                         int E, int nchunks,
                                                         int32_t* __restrict__ chunk_base,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ zero_claims) {
  __shared__ int part[16][64];
  if (zero_claims && blockIdx.x == 0 && threadIdx.x < kClaimInts) zero_claims[threadIdx.x] = 0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 64 + lane;
  const int per = div_up(nchunks, 16);
  const int c0 = min(nchunks, wave * per), c1 = min(nchunks, c0 + per);
  int sum = 0;
  if (e < E) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) sum += chunk_hist[(size_t)c * E + e];
  }
  part[wave][lane] = sum;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += part[w][lane];
  if (e < E) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) {
      const int v = chunk_hist[(size_t)c * E + e];
      chunk_base[(size_t)c * E + e] = base;
      base += v;
    }
    if (wave == 15) counts[e] = base;
  }
}

// Exclusive scan of counts[0..E) into s_off[0..E] by a block of WAVES wavefronts, PER experts
// per thread (E <= 64 WAVES PER).  Contains barriers: call from every thread of the block.
template <int WAVES, int PER>
__device__ __forceinline__ void block_offsets(const int32_t* __restrict__ counts, int E,
                                              int* s_off) {
  __shared__ int wsum[WAVES];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int v[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    v[i] = e < E ? counts[e] : 0;
    sum += v[i];
  }
  const int inc = wave_inclusive_scan(sum);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int base = inc - sum;
  for (int w = 0; w < wave; ++w) base += wsum[w];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    if (e < E) s_off[e] = base;
    base += v[i];
  }
  if (tid == 64 * WAVES - 1) s_off[E] = base;  // the last thread ends with the total
  __syncthreads();
}

// Rows of the (kept) slots of the chunk this wavefront handles: row = offsets[e] + chunk
// base of e + the rank of the token among the chunk's tokens routed to e (bitmap popcount).
// base(e): the number of rows of e in the chunks before this one.
template <bool HAS_KEEP, bool CAND, class Base>
__device__ __forceinline__ void scatter_chunk(const uint64_t* bm, const int* s_off, Base base,
                                              const int32_t* __restrict__ ids,
                                              const uint8_t* __restrict__ keep, int T, int E,
                                              int k, int c, int nchunks,
                                              int32_t* __restrict__ row_token,
                                              int32_t* __restrict__ slot_to_row,
                                              int32_t* __restrict__ cand_slot) {
  const int lane = threadIdx.x & 63;
  const int t = c * kChunk + lane;
  if (c >= nchunks || t >= T) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j0 = 0; j0 < k; j0 += kBatch) {
    int ev[kBatch], bv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const size_t s = (size_t)t * k + j0 + j;
      ev[j] = load_slot<HAS_KEEP>(ids, keep, s, j0 + j < k);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) bv[j] = (ev[j] != -1 && id_usable(ev[j], E)) ? base(ev[j]) : 0;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (j0 + j >= k) break;
      const size_t s = (size_t)t * k + j0 + j;
      const int e = ev[j];
      if (e != -1 && id_usable(e, E)) {
        const int row = s_off[e] + bv[j] + __popcll(bm[e] & below);
        if (CAND) {
          cand_slot[row] = (int32_t)s;
        } else {
          row_token[row] = t;
          slot_to_row[s] = row;
        }
      } else if (!CAND) {
        slot_to_row[s] = -1;
      }
    }
  }
}

// Every block scans the counts into offsets itself (E <= 1024 values, cheaper than a
// launch of its own); block 0 also writes them out.
template <bool HAS_KEEP, bool CAND>
__global__ __launch_bounds__(64 * kLayoutWaves) void scatter_kernel(
    const int32_t* __restrict__ ids, const uint8_t* __restrict__ keep, int T, int E, int k,
    int nchunks, const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
    int32_t* __restrict__ slot_to_row, int32_t* __restrict__ cand_slot) {
  extern __shared__ uint64_t smem_bm[];
  __shared__ int s_off[kMaxE + 4];
  const int wave = threadIdx.x >> 6;
  const int c = blockIdx.x * kLayoutWaves + wave;
  block_offsets<kLayoutWaves, kMaxE / (64 * kLayoutWaves)>(counts, E, s_off);
  if (blockIdx.x == 0)
    for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = s_off[e];
  uint64_t* bm = smem_bm + (size_t)wave * E;
  build_chunk_bitmap<HAS_KEEP>(bm, ids, keep, T, E, k, c, nchunks);
  const int32_t* cb = chunk_base + (size_t)c * E;
  scatter_chunk<HAS_KEEP, CAND>(bm, s_off, [cb](int e) { return cb[e]; }, ids, keep, T, E, k,
                                c, nchunks, row_token, slot_to_row, cand_slot);
}

// Capacity selection, one block per expert.  Keys (weight bits << 32) | (~token) are
// unique per expert and order like (weight desc, token asc) when compared as unsigned
// integers (weights are >= 0).  An MSD radix select over 8-bit digits finds the
// C-th largest key; every key below it is dropped.
__device__ __forceinline__ uint64_t cap_key(const float* __restrict__ w, int32_t slot, int k) {
  const uint32_t wb = __float_as_uint(w[slot]);
  const uint32_t t = (uint32_t)(slot / k);
  return ((uint64_t)wb << 32) | (uint32_t)(0xFFFFFFFFu - t);
}

constexpr int kCapThreads = 1024;
constexpr int kCapLdsKeys = 12288;  // candidates whose keys are held in LDS (96 KiB)

__global__ __launch_bounds__(kCapThreads) void capacity_select_kernel(
    const int32_t* __restrict__ cand_counts, const int32_t* __restrict__ cand_offsets,
    const int32_t* __restrict__ cand_slot, const float* __restrict__ w, int k, int C,
    uint8_t* __restrict__ keep) {
  __shared__ uint64_t s_keys[kCapLdsKeys];
  __shared__ uint32_t hist[256];
  __shared__ int s_sel, s_need, s_done;
  const int e = blockIdx.x;
  const int cnt = cand_counts[e];
  if (cnt <= C) return;  // block-uniform
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int32_t* slots = cand_slot + cand_offsets[e];
  // keys are built once into LDS when they fit; otherwise every pass rebuilds them
  const bool in_lds = cnt <= kCapLdsKeys;  // block-uniform
  if (in_lds)
    for (int i = tid; i < cnt; i += kCapThreads) s_keys[i] = cap_key(w, slots[i], k);
  auto key_at = [&](int i) { return in_lds ? s_keys[i] : cap_key(w, slots[i], k); };
  uint64_t prefix = 0, mask = 0;
  int need = C;
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < cnt; i += kCapThreads) {
      const uint64_t key = key_at(i);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    // The boundary digit: the largest d with (keys above d) < need <= (keys at or above d).
    // Wavefront 0, lane l holding digits 255 - 4l .. 252 - 4l (descending).
    if (wave == 0) {
      uint32_t h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) h[q] = hist[255 - (4 * lane + q)];
      const int lsum = (int)(h[0] + h[1] + h[2] + h[3]);
      int above = wave_inclusive_scan(lsum) - lsum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (above < need && above + (int)h[q] >= need) {  // exactly one lane and q
          s_sel = 255 - (4 * lane + q);
          s_need = need - above;
          s_done = ((int)h[q] == need - above);
        }
        above += (int)h[q];
      }
    }
    __syncthreads();
    const int sel = s_sel;
    need = s_need;
    const int done = s_done;
    prefix |= (uint64_t)sel << shift;
    mask |= (uint64_t)0xFF << shift;
    if (done) break;  // block-uniform
    // (the barrier at the top of the next pass orders these reads before hist is cleared)
  }
  // keys >= prefix (the lower bits of prefix are zero) are exactly the C largest
  for (int i = tid; i < cnt; i += kCapThreads)
    if (key_at(i) < prefix) keep[slots[i]] = 0;
}

// One token per block: read x[t] once, write it to each of its rows.  NT: the row copies
// are stored with the non-temporal hint (written once, read later by another kernel).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__global__ __launch_bounds__(1024) void gather_kernel(const uint4* __restrict__ x,
                                                      const int32_t* __restrict__ slot_to_row,
                                                      int k, int nvec, uint4* __restrict__ xp) {
  __shared__ int rows[32];
  const int t = blockIdx.x;
  if ((int)threadIdx.x < k) rows[threadIdx.x] = slot_to_row[(size_t)t * k + threadIdx.x];
  __syncthreads();
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    const uint4 d = x[(size_t)t * nvec + v];
    for (int j = 0; j < k; ++j) {
      const int r = rows[j];
      if (r < 0) continue;
      if constexpr (NT)
        __builtin_nontemporal_store(u32x4_t{d.x, d.y, d.z, d.w},
                                    reinterpret_cast<u32x4_t*>(&xp[(size_t)r * nvec + v]));
      else
        xp[(size_t)r * nvec + v] = d;
    }
  }
}

inline size_t bitmap_lds(const moe_problem& p) {
  return (size_t)kLayoutWaves * p.E * sizeof(uint64_t);
}

#ifdef MOE_DEBUG_CHECKS
// Status word of the device-side precondition checks: bit 0 an id outside [0, E), bit 1 an id
// that appears twice among a token's k slots.  Sticky until read (moe_debug_status).
__device__ unsigned int g_debug_status;

__global__ __launch_bounds__(256) void check_ids_kernel(const int32_t* __restrict__ ids, int T,
                                                        int k, int E) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  const int32_t* r = ids + (size_t)t * k;
  unsigned int bad = 0;
  for (int j = 0; j < k; ++j) {
    const int e = r[j];
    if (e < 0 || e >= E) bad |= 1u;
    for (int i = 0; i < j; ++i)
      if (r[i] == e) bad |= 2u;
  }
  if (bad) atomicOr(&g_debug_status, bad);
}
#endif

}  // namespace

static hipError_t launch_chunk_hist(const moe_problem& p, const int32_t* ids,
                                    const uint8_t* keep, int32_t* chunk_hist, hipStream_t s) {
  const int nchunks = div_up(p.T, kChunk);
  dim3 grid(div_up(nchunks, kLayoutWaves));
  if (keep)
    hipLaunchKernelGGL(chunk_hist_kernel<true>, grid, dim3(64 * kLayoutWaves), bitmap_lds(p), s,
                       ids, keep, p.T, p.E, p.k, nchunks, chunk_hist);
  else
    hipLaunchKernelGGL(chunk_hist_kernel<false>, grid, dim3(64 * kLayoutWaves), bitmap_lds(p), s,
                       ids, keep, p.T, p.E, p.k, nchunks, chunk_hist);
  return hipGetLastError();
}

hipError_t launch_layout(const moe_problem& p, const int32_t* ids, const uint8_t* keep,
                         int32_t* chunk_hist, int32_t* chunk_base, int32_t* counts,
                         int32_t* offsets, int32_t* row_token, int32_t* slot_to_row,
                         int32_t* cand_slot, hipStream_t s, int32_t* zero_claims) {
  const int nchunks = div_up(p.T, kChunk);
  hipError_t err = launch_chunk_hist(p, ids, keep, chunk_hist, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(scan_cols_kernel, dim3(div_up(p.E, 64)), dim3(1024), 0, s, chunk_hist, p.E,
                     nchunks, chunk_base, counts, zero_claims);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  dim3 grid(div_up(nchunks, kLayoutWaves));
  const size_t lds = bitmap_lds(p);
#define MOE_SCATTER(HK, CAND)                                                                \
  hipLaunchKernelGGL((scatter_kernel<HK, CAND>), grid, dim3(64 * kLayoutWaves), lds, s, ids,   \
                     keep, p.T, p.E, p.k, nchunks, chunk_base, counts, offsets, row_token,     \
                     slot_to_row, cand_slot)
  if (cand_slot)
    MOE_SCATTER(false, true);
  else if (keep)
    MOE_SCATTER(true, false);
  else
    MOE_SCATTER(false, false);
#undef MOE_SCATTER
  return hipGetLastError();
}

hipError_t launch_capacity_select(const moe_problem& p, const int32_t* cand_counts,
                                  const int32_t* cand_offsets, const int32_t* cand_slot,
                                  const float* topk_w, uint8_t* keep, hipStream_t s) {
  hipLaunchKernelGGL(capacity_select_kernel, dim3(p.E), dim3(kCapThreads), 0, s, cand_counts,
                     cand_offsets, cand_slot, topk_w, p.k, p.capacity, keep);
  return hipGetLastError();
}

hipError_t launch_gather(const moe_problem& p, const void* x, const int32_t* slot_to_row,
                         void* xp, hipStream_t s) {
  const size_t row_bytes = (size_t)p.H * (p.act_dtype == MOE_BF16 ? 2 : 4);
  const int nvec = (int)(row_bytes / 16);
  // one thread per 16-byte vector of a row when a row has at most 1024 of them; past 256 MiB
  // of xp (the size of the last-level cache) the copies are streamed with the
  // non-temporal hint, as in the combine
  const int threads = nvec <= 1024 ? (nvec + 63) / 64 * 64 : 256;
  if ((int64_t)p.T * p.k * (int64_t)row_bytes > ((int64_t)256 << 20))
    hipLaunchKernelGGL(gather_kernel<true>, dim3(p.T), dim3(threads), 0, s, (const uint4*)x,
                       slot_to_row, p.k, nvec, (uint4*)xp);
  else
    hipLaunchKernelGGL(gather_kernel<false>, dim3(p.T), dim3(threads), 0, s, (const uint4*)x,
                       slot_to_row, p.k, nvec, (uint4*)xp);
  return hipGetLastError();
}

#ifdef MOE_DEBUG_CHECKS
hipError_t launch_check_ids(const moe_problem& p, const int32_t* ids, hipStream_t s) {
  hipLaunchKernelGGL(check_ids_kernel, dim3(div_up(p.T, 256)), dim3(256), 0, s, ids, p.T, p.k,
                     p.E);
  return hipGetLastError();
}

hipError_t debug_status_take(uint32_t* out) {
  hipError_t err = hipDeviceSynchronize();
  if (err == hipSuccess) err = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_debug_status), 4);
  const unsigned int zero = 0;
  if (err == hipSuccess) err = hipMemcpyToSymbol(HIP_SYMBOL(g_debug_status), &zero, 4);
  return err;
}
#endif

}  // namespace moe
