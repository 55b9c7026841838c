/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer hot path: one GPU's share of an
 * expert-parallel mixture-of-experts layer.
 *
 *   moe_route        top-k routing + per-expert capacity           (route)
 *   moe_router       router GEMM from the hidden states + grouped top-k + capacity
 *   moe_dispatch     expert-contiguous permutation of token rows   (local dispatch)
 *   moe_expert_ffn   grouped SwiGLU FFN = moe_expert_gate_up + moe_expert_down
 *   moe_combine      weighted sum of each token's expert rows     (combine)
 *   moe_layer        all of the above on one stream
 *   moe_layer_chunked  the layer over chunks of tokens, layouts on a second stream,
 *                    optional shared expert
 *   moe_layer_backward gradients of the layer (x, expert weights, logits, router)
 *
 * The pages describe the operations in prose; each declaration names the passage:
 *   [axolotl]  docs.axolotl.ai "integrations.expert_parallel.args", attribute table
 *              (row `expert_parallel_token_capacity`; function
 *              `validate_expert_parallel_topology`).
 *   [LightLLM] LightLLM PR #1687 page: the PR body's call-order paragraph (top-k in the
 *              logical expert space, `norm_topk_prob`, `experts()` versus
 *              `experts_with_topk()`, expert prefix-sum layout for the grouped GEMM,
 *              `silu_and_mul` after the gate/up GEMM) and the walkthrough table row
 *              "Synchronous prefill and decode execution" (decode reduces expert outputs
 *              into dense output).
 *   [WideEP]   research-vault claim card, "Evidence": pure DP+EP has one communication
 *              pattern, the all-to-all that routes tokens to experts.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers (HBM of the current HIP device), row-major,
 *     contiguous.  `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on `stream` and returns; nothing synchronises the host, nothing
 *     allocates or frees device memory, no state survives between calls.
 *   - The caller owns every buffer, including the workspace `ws` of at least
 *     moe_workspace_bytes(p, op) bytes (256-byte aligned).  Row buffers (row_token, xp,
 *     yp) hold T*k rows: the number of kept assignments N is only known on the device.
 *   - Errors are reported synchronously, before anything is enqueued:
 *       MOE_ERR_INVALID_ARG  NULL required pointer, non-positive sizes, k > E, unknown
 *                            dtype, misaligned pointer, or aliasing: an output buffer (the
 *                            workspace included) whose byte range, sized from the problem as
 *                            documented for each call (row buffers hold T*k rows), overlaps
 *                            an input buffer or another output (inputs may share memory);
 *       MOE_ERR_UNSUPPORTED  a valid problem the kernels do not handle (see
 *                            moe_problem_check);
 *       MOE_ERR_WORKSPACE    ws_bytes < moe_workspace_bytes(p, op);
 *       MOE_ERR_HIP          a launch failed (hipGetLastError after enqueueing).
 *     No call ever falls back to another implementation.
 *   - Device-side preconditions (not checked in the release library): logits finite;
 *     caller-supplied ids in [0, E) and distinct within a token.  The debug library
 *     (libmoe_debug.so, built with MOE_DEBUG_CHECKS) checks the ids wherever a call takes
 *     them from the caller (moe_dispatch, moe_layer_backward), treats a slot whose id lies
 *     outside [0, E) as dropped instead of indexing with it, and reports violations through
 *     moe_debug_status.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE = 3,
  MOE_ERR_HIP = 4
} moe_status;

/* MOE_FP8 (weights only, with bf16 activations): [LightLLM] walkthrough table row
 * "Grouped MoE kernel support" (FP8 grouped GEMMs over the prefix-sum layout, SwiGLU
 * fused with quantisation, UE8M0 scale tests) and the review comment on the UE8M0 test
 * (block scales are exact powers of two, 2^-8 in its case).  Format: OCP E4M3 codes
 * (largest finite 448, round to nearest even, saturating) with one UE8M0 scale byte
 * (value 2^(byte-127)) per 32 consecutive elements along the reduction dimension; the
 * scale of a block is the smallest power of two 2^e with max|x| <= 448 * 2^e (2^0 for an
 * all-zero block). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8 = 2 } moe_dtype;

/* Problem description.  T tokens of width H, E experts, top-k, SwiGLU width I. */
typedef struct {
  int32_t T, H, E, k, I;
  /* Max (token, expert) assignments per expert per call; <= 0 means no cap
   * ([axolotl] `expert_parallel_token_capacity`, None = no cap). */
  int32_t capacity;
  /* 1: the top-k weights are renormalised to sum to 1 ([LightLLM] `norm_topk_prob`);
   * 0: they are the plain softmax probabilities over all E experts. */
  int32_t renormalize;
  int32_t act_dtype; /* moe_dtype of x, xp, yp, y and (unless w_dtype is FP8) of the
                        intermediate activation */
  int32_t w_dtype;   /* moe_dtype of the expert weights (MOE_FP8 needs act MOE_BF16) */
} moe_problem;

typedef enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_DISPATCH = 1,
  MOE_OP_FFN = 2, /* moe_expert_ffn; FP8 problems: also moe_expert_gate_up(_gather) */
  MOE_OP_COMBINE = 3,
  MOE_OP_LAYER = 4,
  MOE_OP_ROUTER = 5, /* moe_router: split-K partial logits (+ capacity scratch) */
  MOE_OP_BACKWARD = 6 /* moe_layer_backward (with the router and the yp recompute) */
} moe_op;

typedef enum { MOE_W_GATE_UP = 0, MOE_W_DOWN = 1 } moe_weight_set;

/* Text for a status code (static storage). */
const char* moe_status_str(int status);

/* Debug library only ([axolotl] `validate_expert_parallel_topology`: what the kernels cannot
 * handle is reported, never run another way): waits for the current device, writes the
 * sticky status word of its precondition checks to *status and clears it.  Bit 0: an expert
 * id outside [0, E) was passed; bit 1: a token's k ids were not distinct.  The release
 * library sets *status = 0 and returns MOE_ERR_UNSUPPORTED; MOE_ERR_INVALID_ARG if status
 * is NULL. */
int moe_debug_status(uint32_t* status);

/* Host-only validation of a problem ([axolotl] `validate_expert_parallel_topology`:
 * layouts the kernels do not handle are rejected up front, never run another way).
 * Returns MOE_OK, MOE_ERR_INVALID_ARG (p NULL, T/H/E/k/I < 1, k > E, dtype unknown) or
 * MOE_ERR_UNSUPPORTED: E > 1024, k > 32, act_dtype != w_dtype (except FP8 weights with
 * bf16 activations), H or I not a multiple of 64 (bf16), 128 (FP8) or 8 (f32),
 * T*k >= 2^31. */
int moe_problem_check(const moe_problem* p);

/* Workspace bytes that `op` needs for problem p (0 if p is invalid). */
size_t moe_workspace_bytes(const moe_problem* p, int op);

/* ---------------------------------------------------------------------------------
 * Expert weights.  The natural layout is W_gate, W_up: [E, H, I] and W_down: [E, I, H]
 * (row-major, y = x W).  The kernels read a packed copy in which every 32-column by
 * 16-row block of a weight matrix is one contiguous 1 KiB matrix-core operand (the
 * reduction dimension contiguous in 8-element runs, as the pages' grouped GEMMs take
 * their weights "nt").  Packing is a one-time step when weights are loaded, like any
 * checkpoint layout conversion; the packed buffers stay resident and are what
 * moe_expert_ffn and moe_layer read.
 *
 * moe_packed_bytes: size of one packed set (MOE_W_GATE_UP holds gate and up).
 * moe_pack_weights: writes packed_gate_up (E*2*H*I elements) and packed_down
 *   (E*I*H elements) from the natural layout; elements are copied bit for bit.
 *   For f32 problems the packed layout is the natural layout.
 *   For FP8 problems the natural layout is bf16 and packing quantises: every block of
 *   32 elements along the reduction dimension (H for gate/up, I for down) of one output
 *   column gets its UE8M0 scale and E4M3 codes, as moe_quantize_fp8 would compute for
 *   that column; the packed buffer holds the codes in matrix-core operand order followed
 *   (at a 256-byte boundary) by the scale bytes.
 * --------------------------------------------------------------------------------- */
size_t moe_packed_bytes(const moe_problem* p, int which);
int moe_pack_weights(const moe_problem* p, const void* w_gate, const void* w_up,
                     const void* w_down, void* packed_gate_up, void* packed_down,
                     void* stream);

/* ---------------------------------------------------------------------------------
 * moe_route -- [LightLLM] call-order paragraph: top-k chosen in the logical expert
 * space, weights optionally renormalised; [axolotl] capacity row: at most `capacity`
 * assignments per expert, the lowest-weight excess dropped.
 *
 *   logits   [T, E] f32   router logits (input, finite)
 *   topk_ids [T, k] i32   expert ids, slot order = logit descending, ties to the
 *                         lower expert id
 *   topk_w   [T, k] f32   softmax weights of the chosen experts (renormalised to sum
 *                         to 1 if p->renormalize); computed with a specified fp32
 *                         arithmetic so they are reproducible bit for bit
 *   keep     [T, k] u8    1 = kept, 0 = dropped by the capacity (all 1 without a cap).
 *                         Order for dropping: weight ascending, ties: higher token
 *                         index dropped first.  Dropped slots keep their weight in
 *                         topk_w; they are not re-routed.
 * --------------------------------------------------------------------------------- */
int moe_route(const moe_problem* p, const float* logits, int32_t* topk_ids, float* topk_w,
              uint8_t* keep, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_route_grouped -- [LightLLM] call-order paragraph: `experts()` does grouped top-k
 * inside the layer.  The pages do not give the group rule; this is its plain reading:
 * the E experts form n_group groups of E / n_group consecutive ids, a group's score is
 * its largest logit, the topk_group best groups are taken (ties to the lower group
 * index), and the top-k of the experts in the taken groups are selected (order, ties,
 * weights, renormalisation and capacity exactly as moe_route).  n_group = 1 (or
 * topk_group = n_group) is moe_route.
 * MOE_ERR_INVALID_ARG unless 1 <= topk_group <= n_group <= 64, n_group divides E and
 * k <= topk_group * E / n_group.  Workspace: moe_workspace_bytes(p, MOE_OP_ROUTE).
 * --------------------------------------------------------------------------------- */
int moe_route_grouped(const moe_problem* p, const float* logits, int32_t n_group,
                      int32_t topk_group, int32_t* topk_ids, float* topk_w, uint8_t* keep,
                      void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_router -- the routing front-end from the hidden states ([LightLLM] call-order
 * paragraph: the layer's `experts()` computes its routing itself): a linear gate without
 * bias, logits[t, e] = sum_h x[t, h] * w_router[e, h] (bf16 operands, fp32 accumulation
 * on the matrix cores), then the selection of moe_route_grouped and the capacity, in one
 * launch (plus the capacity kernels when capacity > 0).
 *   x        [T, H] bf16      hidden states (16-byte aligned)
 *   w_router [E, H] bf16      gate weights, one row per expert (the layout of a
 *                             bias-free linear layer's weight; 16-byte aligned)
 *   logits   [T, E] f32 or NULL: receives the logits (not needed by the selection)
 *   topk_ids, topk_w, keep    as moe_route
 * The selection is taken on the fp32 logits this call computes: the GEMM is split along
 * H into S equal slices (S chosen from T and H so that the grid fills the chip) whose
 * partial sums go to the workspace and are added in slice order by the selection kernel.
 * Workspace: moe_workspace_bytes(p, MOE_OP_ROUTER).
 * MOE_ERR_UNSUPPORTED unless act_dtype is bf16, E <= 256 and E is a multiple of 16;
 * MOE_ERR_INVALID_ARG for the group arguments as in moe_route_grouped.
 * --------------------------------------------------------------------------------- */
int moe_router(const moe_problem* p, const void* x, const void* w_router, int32_t n_group,
               int32_t topk_group, float* logits, int32_t* topk_ids, float* topk_w,
               uint8_t* keep, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_dispatch -- [LightLLM] expert prefix-sum layout (`use_psum_layout`); [WideEP]:
 * on one GPU the dispatch all-to-all becomes this permutation.  Accepts caller routing
 * ([LightLLM] `experts_with_topk`).
 *
 *   x           [T, H]    act dtype  token rows
 *   topk_ids    [T, k]    i32
 *   keep        [T, k]    u8 or NULL (NULL: all kept)
 *   counts      [E]       i32  kept assignments per expert            (output)
 *   offsets     [E+1]     i32  exclusive scan of counts, offsets[E]=N (output)
 *   row_token   [T*k]     i32  token of row r for r < N; rows of an expert are
 *                              contiguous and in ascending token order (output)
 *   slot_to_row [T, k]    i32  row of slot (t, j), -1 if dropped        (output)
 *   xp          [T*k, H]  act dtype  xp[r] = x[row_token[r]] for r < N  (output), or
 *                              NULL: the layout only, no row copy (the rows are then read
 *                              through row_token by moe_expert_gate_up_gather)
 * All integer outputs are deterministic (no atomics-order effects).
 * --------------------------------------------------------------------------------- */
int moe_dispatch(const moe_problem* p, const void* x, const int32_t* topk_ids,
                 const uint8_t* keep, int32_t* counts, int32_t* offsets, int32_t* row_token,
                 int32_t* slot_to_row, void* xp, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * Grouped SwiGLU expert FFN over the prefix-sum layout ([LightLLM]: grouped GEMM, then
 * `silu_and_mul`).  For each expert e and each of its rows r in
 * [offsets[e], offsets[e+1]):
 *   a[r]  = silu(xp[r] Wg[e]) * (xp[r] Wu[e]),   silu(z) = z / (1 + exp(-z))
 *   yp[r] = a[r] Wd[e]
 * fp32 accumulation; `a` and yp are stored in the activation dtype.  offsets are read
 * on the device (no host synchronisation); rows >= offsets[E] are not touched.
 *
 *   xp [T*k, H], a [T*k, I], yp [T*k, H] (act dtype); offsets [E+1] i32;
 *   packed_gate_up / packed_down from moe_pack_weights.
 * moe_expert_ffn keeps `a` in the workspace; the two halves are also callable alone and
 * need no workspace (their ws / ws_bytes arguments are ignored and may be NULL / 0).
 *
 * moe_expert_gate_up_gather is moe_expert_gate_up with the dispatch row copy folded into
 * the operand loads: row r of the layout is read as x[row_token[r]] (x [T, H], row_token
 * from moe_dispatch), so xp is never materialised.  Same result, bit for bit.
 *
 * FP8 weights (w_dtype MOE_FP8): the bf16 input rows are first quantised per row as by
 * moe_quantize_fp8 (into the workspace: these calls then need ws of
 * moe_workspace_bytes(p, MOE_OP_FFN) bytes), the products use the E4M3 codes scaled by
 * their UE8M0 block scales with fp32 accumulation, and the intermediate activation `a` is
 * stored quantised the same way: E4M3 codes [T*k, I] (row r at a + r*I) followed, at the
 * next 256-byte boundary, by the scale bytes [T*k, I/32].  Its size is
 * align256(T*k*I) + T*k*I/32 bytes.  yp stays bf16.
 * --------------------------------------------------------------------------------- */
int moe_expert_ffn(const moe_problem* p, const void* xp, const int32_t* offsets,
                   const void* packed_gate_up, const void* packed_down, void* yp, void* ws,
                   size_t ws_bytes, void* stream);
int moe_expert_gate_up(const moe_problem* p, const void* xp, const int32_t* offsets,
                       const void* packed_gate_up, void* a, void* ws, size_t ws_bytes,
                       void* stream);
int moe_expert_gate_up_gather(const moe_problem* p, const void* x, const int32_t* row_token,
                              const int32_t* offsets, const void* packed_gate_up, void* a,
                              void* ws, size_t ws_bytes, void* stream);
int moe_expert_down(const moe_problem* p, const void* a, const int32_t* offsets,
                    const void* packed_down, void* yp, void* ws, size_t ws_bytes,
                    void* stream);

/* ---------------------------------------------------------------------------------
 * moe_quantize_fp8 -- the per-block activation quantisation of the FP8 path (same
 * passages as MOE_FP8): for each row of x [rows, cols] bf16 and each block b of 32
 * columns, scales[row, b] = the UE8M0 byte of the block and codes[row, c] = the E4M3
 * code of x[row, c] / 2^(scale-127), rounded to nearest even, saturating at 448.
 *   codes [rows, cols] u8 (16-byte aligned), scales [rows, cols/32] u8.
 * rows = 0 enqueues nothing.  MOE_ERR_INVALID_ARG: rows < 0, cols not a positive
 * multiple of 32, NULL or misaligned pointers.
 * --------------------------------------------------------------------------------- */
int moe_quantize_fp8(const void* x, int64_t rows, int32_t cols, uint8_t* codes,
                     uint8_t* scales, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_combine -- [LightLLM] walkthrough, "Synchronous prefill and decode execution":
 * expert outputs are reduced back into dense token order.
 *   y[t] = sum over j = 0..k-1 with slot_to_row[t,j] >= 0 of topk_w[t,j] * yp[row]
 * summed in fp32 in slot order (deterministic, no atomics), stored in the act dtype.
 * A token whose slots were all dropped gets 0.
 *   yp [T*k, H], topk_w [T, k] f32, slot_to_row [T, k] i32, y [T, H].
 * --------------------------------------------------------------------------------- */
int moe_combine(const moe_problem* p, const void* yp, const float* topk_w,
                const int32_t* slot_to_row, void* y, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_layer -- route, capacity, dispatch, FFN and combine in one call on one stream (the
 * dispatch builds the layout only and gate/up gathers the token rows itself).
 * x [T, H], logits [T, E] f32, packed weights, y [T, H].  The routing outputs are
 * optional: pass NULL to keep them in the workspace, or buffers of the shapes above to
 * receive them.
 * --------------------------------------------------------------------------------- */
int moe_layer(const moe_problem* p, const void* x, const float* logits,
              const void* packed_gate_up, const void* packed_down, void* y,
              int32_t* topk_ids, float* topk_w, uint8_t* keep, int32_t* counts,
              int32_t* offsets, int32_t* row_token, int32_t* slot_to_row, void* ws,
              size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_layer_static -- moe_layer for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments without a workspace; the workspace is a device array inside the library of
 * moe_layer_static_max_bytes() bytes (32 MiB), one per GPU the library runs on, held until
 * the process ends.  Nothing is allocated or freed by the call.  Every call on a GPU shares
 * that GPU's array, which keeps the last call's contents (the layer writes everything it
 * later reads, so nothing needs clearing): calls that overlap in time on one GPU (other
 * streams, other host threads) race and give undefined results.  MOE_ERR_WORKSPACE if
 * moe_workspace_bytes(p, MOE_OP_LAYER) exceeds the array (e.g. decode batches of a few
 * hundred tokens fit at DeepSeek-V3 width); otherwise errors and results as moe_layer,
 * bit for bit.
 * --------------------------------------------------------------------------------- */
size_t moe_layer_static_max_bytes(void);
int moe_layer_static(const moe_problem* p, const void* x, const float* logits,
                     const void* packed_gate_up, const void* packed_down, void* y,
                     int32_t* topk_ids, float* topk_w, uint8_t* keep, int32_t* counts,
                     int32_t* offsets, int32_t* row_token, int32_t* slot_to_row, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_layer_chunked -- moe_layer over chunks of tokens, with the next chunk's layout
 * built on a second stream while the current chunk's experts run, and an optional shared
 * expert ([LightLLM] PR body: the chunked expanded forward bounds each call's temporary
 * rows (at most 32K there); the shared expert's output is added in the combine, its
 * computation overlapped with the routed experts on the other stream).
 *
 * Routing and the capacity are computed once over all T tokens on `stream` (so the result
 * does not depend on the chunking: y equals moe_layer's bit for bit without a shared
 * expert).  Then for each chunk of up to chunk_tokens tokens: its expert-contiguous layout
 * (and the shared expert's rows) on `aux_stream`, the routed gate/up, down and the
 * combine (which adds the shared rows last, in fp32, before the one rounding) on
 * `stream`.  Two layout sets alternate; events order the two streams, so work issued
 * later on `stream` sees the whole result.  aux_stream NULL (or equal to stream): all on
 * `stream`.  Events are created and released inside the call (no device memory).
 *
 *   shared       NULL, or the shared expert: its intermediate width I and its weights
 *                packed by moe_pack_weights for the problem {T, H, E = 1, k = 1, I,
 *                same dtypes}; y[t] = routed combine + SwiGLU_shared(x[t]).
 *   chunk_tokens >= 1 (clamped to T); the workspace grows with it, not with T (except
 *                for the [T, k] routing results).
 * Workspace: moe_layer_chunked_workspace_bytes(p, chunk_tokens, shared ? shared->I : 0)
 * (0 if the arguments are invalid).  Errors as moe_layer; MOE_ERR_INVALID_ARG for
 * chunk_tokens < 1 or a NULL shared weight; the shared problem must pass
 * moe_problem_check (e.g. I a multiple of 64 for bf16).
 * --------------------------------------------------------------------------------- */
typedef struct {
  int32_t I;                  /* the shared expert's intermediate width */
  const void* packed_gate_up; /* moe_pack_weights output for {T, H, 1, 1, I} */
  const void* packed_down;
} moe_shared_expert;

size_t moe_layer_chunked_workspace_bytes(const moe_problem* p, int32_t chunk_tokens,
                                         int32_t shared_I);
int moe_layer_chunked(const moe_problem* p, const void* x, const float* logits,
                      const void* packed_gate_up, const void* packed_down,
                      const moe_shared_expert* shared, int32_t chunk_tokens, void* y, void* ws,
                      size_t ws_bytes, void* stream, void* aux_stream);

/* ---------------------------------------------------------------------------------
 * Backward pass -- [axolotl] attribute table, row `expert_parallel_save_dispatch`: the
 * backward reuses the forward's routing (top-k and split counts are always saved) and the
 * dispatch rows (here: gathered again from x through the saved row_token).  Gradients of
 * the forward above (route -> capacity -> layout -> SwiGLU experts -> combine) for an
 * upstream gradient dy; the selection itself carries no gradient.
 *
 * moe_expert_gate_up_gather_gu: moe_expert_gate_up_gather (bf16) that also stores the
 *   pre-activations for the backward: gu [T*k, 2I] bf16, row r of the layout holding
 *   g = x W_gate[e] and u = x W_up[e] in 32-column blocks that alternate (columns 64 b ..
 *   64 b + 31: g columns 32 b .., the next 32: u columns 32 b ..), rounded from the same
 *   fp32 accumulators that give a (a is bit for bit that of moe_expert_gate_up_gather).
 *   Memory against time: the backward then skips its recompute of g|u.  Needs no
 *   workspace.  MOE_ERR_UNSUPPORTED as moe_layer_backward (bf16, H % 128 == 0,
 *   H <= 8192); MOE_ERR_INVALID_ARG for NULL or misaligned pointers.
 *
 * moe_pack_weights_backward: the backward's operands, one-time like moe_pack_weights,
 *   from the natural bf16 weights: packed_bwd_gate_up (moe_packed_bytes(p,
 *   MOE_W_GATE_UP) bytes) holds [W_gate | W_up]^T, packed_bwd_down (moe_packed_bytes(p,
 *   MOE_W_DOWN) bytes) holds W_down^T.
 *
 * moe_layer_backward:
 *   x [T, H] bf16, logits [T, E] f32 (read only when p->renormalize == 0),
 *   w_router [E, H] bf16 or NULL: the gate of moe_router (then dw_router is written and
 *     dx includes the router's path),
 *   packed_gate_up / packed_down: the forward's packed weights (packed_down is read only
 *     when yp is NULL), packed_bwd_*: from moe_pack_weights_backward,
 *   saved: the forward's routing outputs, yp [T*k, H] bf16: the forward's expert outputs
 *     (moe_expert_down), or NULL to recompute them,
 *   gu [T*k, 2I] bf16: the forward's pre-activations from moe_expert_gate_up_gather_gu,
 *     or NULL to recompute them (one grouped GEMM over the packed gate/up weights; the
 *     saved ones have the same bits, so the gradients do not depend on the choice),
 *   dy [T, H] bf16.
 * Outputs (grads): dx [T, H] bf16; dw_gate, dw_up [E, H, I] and dw_down [E, I, H] f32
 *   (zero for experts without rows); dlogits [T, E] f32; dtopk_w [T, k] f32 or NULL;
 *   dw_router [E, H] f32 (with w_router).
 * Arithmetic: bf16 operands, fp32 accumulation; the intermediate gradients (dyp, da,
 *   [dg | du], dxp) and the recomputed g, u, a are stored in bf16.
 * MOE_ERR_UNSUPPORTED unless act and weight dtypes are bf16, H % 128 == 0, H <= 8192 (and,
 * with a router, E % 64 == 0).  Workspace: moe_workspace_bytes(p, MOE_OP_BACKWARD).
 * --------------------------------------------------------------------------------- */
typedef struct {
  const int32_t* topk_ids;    /* [T, k] */
  const float* topk_w;        /* [T, k] */
  const int32_t* offsets;     /* [E + 1] */
  const int32_t* row_token;   /* [T * k] */
  const int32_t* slot_to_row; /* [T, k], -1 for dropped slots */
} moe_saved_routing;

typedef struct {
  void* dx;         /* [T, H] bf16 */
  float* dw_gate;   /* [E, H, I] */
  float* dw_up;     /* [E, H, I] */
  float* dw_down;   /* [E, I, H] */
  float* dlogits;   /* [T, E] */
  float* dtopk_w;   /* [T, k] or NULL */
  float* dw_router; /* [E, H], with a router */
} moe_grads;

int moe_pack_weights_backward(const moe_problem* p, const void* w_gate, const void* w_up,
                              const void* w_down, void* packed_bwd_gate_up,
                              void* packed_bwd_down, void* stream);
int moe_expert_gate_up_gather_gu(const moe_problem* p, const void* x, const int32_t* row_token,
                                 const int32_t* offsets, const void* packed_gate_up, void* a,
                                 void* gu, void* stream);
int moe_layer_backward(const moe_problem* p, const void* x, const float* logits,
                       const void* w_router, const void* packed_gate_up,
                       const void* packed_down, const void* packed_bwd_gate_up,
                       const void* packed_bwd_down, const moe_saved_routing* saved,
                       const void* yp, const void* gu, const void* dy,
                       const moe_grads* grads, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
