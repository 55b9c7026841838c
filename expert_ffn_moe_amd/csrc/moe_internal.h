// Internal launchers of the MoE hot-path kernels (gfx950).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Tokens per routing chunk: one wavefront, one bit per token in a 64-bit mask.
constexpr int kChunk = 64;
// Largest expert count the kernels handle (moe_problem_check).
constexpr int kMaxE = 1024;
// Rows per M tile of the prefill grouped GEMM.
constexpr int kPrefillBM = 128;

__host__ __device__ inline int div_up(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t div_up64(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Bump allocator over a caller-provided workspace (sizes are rounded to 256 bytes).
struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t count) {
    T* p = base ? reinterpret_cast<T*>(base + used) : nullptr;
    used += align256(count * sizeof(T));
    return p;
  }
};

// Scratch of the routing/dispatch pipeline.
struct RankScratch {
  int32_t* chunk_hist;   // [nchunks, E]
  int32_t* chunk_base;   // [nchunks, E]
  int32_t* cand_counts;  // [E]      (capacity only)
  int32_t* cand_offsets; // [E + 1]  (capacity only)
  int32_t* cand_slot;    // [T * k]  (capacity only)
};
RankScratch carve_rank(Carve& c, const moe_problem& p, bool with_capacity);

// ---- route.hip
// Top-k (group-limited when 1 < n_group and topk_group < n_group) from fp32 logits.
hipError_t launch_route(const moe_problem& p, const float* logits, int n_group, int topk_group,
                        int32_t* ids, float* w, uint8_t* keep, hipStream_t s);
// Router front-end: logits = x W_r^T (bf16, W_r [E, H]) as `split` partial planes
// [split][T][E] f32 in `part` (rows per block, split of H chosen by router_plan), then the
// selection of their in-order sum; the summed logits are also written if not NULL.
struct RouterPlan {
  int rows;   // tokens per block: 64, 128 or 256
  int split;  // slices of H (a divisor of H / 64)
};
bool router_supported(const moe_problem& p);
// d logits [T, E] from d topk_w (0 on dropped slots); logits are read only without
// renormalisation.
hipError_t launch_route_bwd(const moe_problem& p, const float* logits, const int32_t* ids,
                            const float* w, const float* dw, float* dl, hipStream_t s);
RouterPlan router_plan(const moe_problem& p);
hipError_t launch_router(const moe_problem& p, const void* x, const void* wr, int n_group,
                         int topk_group, float* part, float* logits, int32_t* ids, float* w,
                         uint8_t* keep, hipStream_t s);

// ---- dispatch.hip
// The expert layout of the (kept) slots: counts, offsets = their exclusive scan (both written
// out), then the row of each kept slot (stable: rows ascend in token index within an
// expert).  If cand_slot != NULL the rows index the slot list cand_slot (capacity
// candidates) instead of writing row_token / slot_to_row.  Three launches: the per-chunk
// histogram, its column scan and the scatter (chunk_hist, chunk_base: [nchunks, E] scratch).
// zero_claims, if not NULL, receives kClaimInts zeros (the layer's GEMM work counters) from
// the column scan.
hipError_t launch_layout(const moe_problem& p, const int32_t* ids, const uint8_t* keep,
                         int32_t* chunk_hist, int32_t* chunk_base, int32_t* counts,
                         int32_t* offsets, int32_t* row_token, int32_t* slot_to_row,
                         int32_t* cand_slot, hipStream_t s, int32_t* zero_claims = nullptr);
// Capacity: per overflowing expert, radix-select the top-C keys and clear keep for the rest.
hipError_t launch_capacity_select(const moe_problem& p, const int32_t* cand_counts,
                                  const int32_t* cand_offsets, const int32_t* cand_slot,
                                  const float* topk_w, uint8_t* keep, hipStream_t s);
#ifdef MOE_DEBUG_CHECKS
// Debug builds: checks caller-supplied ids ([0, E), distinct within a token) into the status
// word; debug_status_take waits for the device, reads the word and clears it.
hipError_t launch_check_ids(const moe_problem& p, const int32_t* ids, hipStream_t s);
hipError_t debug_status_take(uint32_t* out);
#endif
// Row gather xp[slot_to_row[t, j]] = x[t].
hipError_t launch_gather(const moe_problem& p, const void* x, const int32_t* slot_to_row,
                         void* xp, hipStream_t s);

// ---- combine.hip
// shared: NULL, or the shared expert's output rows [T, H] (act dtype), added last.
hipError_t launch_combine(const moe_problem& p, const void* yp, const float* w,
                          const int32_t* slot_to_row, const void* shared, void* y,
                          hipStream_t s);
// off[0] = 0, off[1] = n (the layout of a one-expert problem over n rows).
hipError_t launch_one_expert_offsets(int32_t* off, int n, hipStream_t s);

// ---- backward.hip
hipError_t launch_combine_bwd(const moe_problem& p, const void* dy, const void* yp,
                              const float* w, const int32_t* slot_to_row, void* dyp, float* dw,
                              hipStream_t s);
// SwiGLU backward from g|u and da (both [T*k, .] in the layout): dgu (row-major, gu's
// interleaving) and, in the padded layout of poff / npad (launch_pad_offsets with gran 64),
// dguT packed like launch_transpose_pad's packed form and aT plain.
hipError_t launch_swiglu_bwd(const moe_problem& p, const void* gu, const void* da,
                             const int32_t* offsets, const int32_t* poff, int64_t npad, void* dgu,
                             void* dguT, void* aT, hipStream_t s);
// poff[e]: the exclusive scan of the counts rounded up to a multiple of gran (16 or 64).
hipError_t launch_pad_offsets(const int32_t* offsets, int E, int gran, int32_t* poff,
                              hipStream_t s);
// [rows, C] bf16 (rows through row_map if not NULL) -> [C, npad], each expert's rows at
// columns poff[e] .. (a multiple of 64), padding columns zeroed; C % 64 == 0, npad % 64 == 0.
// packed: dst in matrix-core operand order ([C / 32][npad / 16] blocks of 1 KiB, like the
// packed down weights with K = npad) instead of row-major.
hipError_t launch_transpose_pad(const void* src, const int32_t* row_map, const int32_t* offsets,
                                const int32_t* poff, int E, int C, int64_t npad, bool packed,
                                void* dst, hipStream_t s);
hipError_t launch_f32_to_bf16(const float* in, int64_t n, void* out, hipStream_t s);

// ---- pack.hip
hipError_t launch_pack(const moe_problem& p, const void* wg, const void* wu, const void* wd,
                       void* packed_gu, void* packed_d, hipStream_t s);
hipError_t launch_pack_backward(const moe_problem& p, const void* wg, const void* wu,
                                const void* wd, void* packed_bwd_gu, void* packed_bwd_d,
                                hipStream_t s);
hipError_t launch_pack_plain(int E, int K, int N, const void* w, void* packed, hipStream_t s);

// ---- ffn_bf16.hip / ffn_f32.hip
// The decode-shaped kernels (few rows per expert) or the prefill ones: decided from the
// whole problem (a chunked layer decides once, so every chunk uses the same kernels).
bool ffn_use_decode(const moe_problem& p);
// Gate/up over the layout's rows: row r reads xs[r] (xp), or xs[row_token[r]] (token rows
// x) when row_token is not NULL.  gu, if not NULL, receives the pre-activations [rows, 2I]
// exactly as launch_gemm_bf16 over the packed gate/up weights computes them.
// claim, if not NULL: 8 work-item counters of the prefill kernel (one per XCD), zero at
// launch; the blocks then take items dynamically instead of round-robin.
hipError_t launch_gate_up_bf16(const moe_problem& p, const void* xs, const int32_t* row_token,
                               const int32_t* offsets, const void* packed_gu, void* a, void* gu,
                               bool decode, hipStream_t s, int* claim = nullptr);
hipError_t launch_down_bf16(const moe_problem& p, const void* a, const int32_t* offsets,
                            const void* packed_d, void* yp, bool decode, hipStream_t s,
                            int* claim = nullptr);
// The work-item counters of one layer call: gate/up's 8, then down's 8.
constexpr int kClaimInts = 16;
// Plain grouped GEMM out[r] = A[r or row_token[r]] B[e] with B packed like the down weights
// (K % 64 == 0 for the prefill kernel, K % 32 for the decode one; Nout % 64 == 0).
hipError_t launch_gemm_bf16(int E, const void* A, const int32_t* row_token,
                            const int32_t* offsets, const void* packed_b, void* out, int K,
                            int Nout, bool decode, hipStream_t s);
// Weight gradients on the matrix cores: out[e][m][n] = sum_k AT[m][k] BT[n][k] over expert
// e's rows [poff[e], poff[e + 1]) (a multiple of 64, zero-padded); Ncols % 64 == 0.  AT is
// row-major [M][npad]; BT is [Ncols][npad] in the packed operand order of
// launch_transpose_pad(packed = true).
hipError_t launch_wgrad_bf16(const void* AT, const void* BT, const int32_t* poff, int E, int M,
                             int Ncols, int64_t npad, bool gu_split, float* out, float* out2,
                             hipStream_t s);
hipError_t launch_gate_up_f32(const moe_problem& p, const float* xs, const int32_t* row_token,
                              const int32_t* offsets, const float* wg, const float* wu, float* a,
                              hipStream_t s);
hipError_t launch_down_f32(const moe_problem& p, const float* a, const int32_t* offsets,
                           const float* wd, float* yp, hipStream_t s);

// ---- quant_fp8.hip / ffn_fp8.hip (FP8 E4M3 operands, UE8M0 scales per 32 along K)
size_t fp8_packed_code_bytes(int E, int K, int N, int nmat);
size_t fp8_packed_scale_bytes(int E, int K, int N, int nmat);
hipError_t launch_pack_fp8(const moe_problem& p, const void* wg, const void* wu, const void* wd,
                           void* packed_gu, void* packed_d, hipStream_t s);
// bf16 rows [rows, K] -> codes [rows, K], scales [rows, K / 32]; rows >= *row_limit
// skipped if row_limit is not NULL (a device pointer).
hipError_t launch_quant_rows(const void* in, int64_t rows, int K, const int32_t* row_limit,
                             uint8_t* codes, uint8_t* scales, hipStream_t s);
// Gate/up on quantised rows (xq/xs; token rows through row_token if not NULL) -> the
// quantised intermediate (aq [rows, I], as [rows, I / 32]); down -> yp (bf16).
hipError_t launch_gate_up_fp8(const moe_problem& p, const uint8_t* xq, const uint8_t* xs,
                              const int32_t* row_token, const int32_t* offsets,
                              const void* packed_gu, uint8_t* aq, uint8_t* as, hipStream_t s);
hipError_t launch_down_fp8(const moe_problem& p, const uint8_t* aq, const uint8_t* as,
                           const int32_t* offsets, const void* packed_d, void* yp,
                           hipStream_t s);

}  // namespace moe
