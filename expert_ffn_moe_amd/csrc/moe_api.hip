// C ABI entry points: argument checks, workspace carving and kernel sequencing.  Every
// step of the path runs in the kernels of this library; there is no other implementation
// to fall back to.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>

#include "moe_internal.h"

namespace moe {

RankScratch carve_rank(Carve& c, const moe_problem& p, bool with_capacity) {
  const size_t nchunks = (size_t)div_up(p.T, kChunk);
  RankScratch r{};
  r.chunk_hist = c.take<int32_t>(nchunks * p.E);
  r.chunk_base = c.take<int32_t>(nchunks * p.E);
  if (with_capacity) {
    r.cand_counts = c.take<int32_t>(p.E);
    r.cand_offsets = c.take<int32_t>((size_t)p.E + 1);
    r.cand_slot = c.take<int32_t>((size_t)p.T * p.k);
  }
  return r;
}

}  // namespace moe

using namespace moe;

namespace {

size_t elem_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }  // activations: bf16 unless f32

bool is_fp8(const moe_problem& p) { return p.w_dtype == MOE_FP8; }

// Quantised activation rows: E4M3 codes [rows, cols] then UE8M0 scale bytes [rows, cols/32]
// at the next 256-byte boundary.
size_t q_rows_bytes(size_t rows, size_t cols) { return align256(rows * cols) + rows * (cols / 32); }
uint8_t* q_scales(void* q, size_t rows, size_t cols) {
  return static_cast<uint8_t*>(q) + align256(rows * cols);
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Workspace of the FFN: the intermediate activation (moe_expert_ffn and moe_layer; the
// split calls take it as an argument), and for FP8 problems the quantised input rows
// (needed by every gate/up call).
struct FfnScratch {
  void* a;
  void* xq;  // FP8: codes + scales of up to T*k input rows
};
FfnScratch carve_ffn(Carve& c, const moe_problem& p) {
  FfnScratch f{};
  const size_t tk = (size_t)p.T * p.k;
  if (is_fp8(p)) {
    f.a = c.take<char>(q_rows_bytes(tk, p.I));
    f.xq = c.take<char>(q_rows_bytes(tk, p.H));
  } else {
    f.a = c.take<char>(tk * p.I * elem_bytes(p.act_dtype));
  }
  return f;
}

// ---- chunked layer: the whole layer's routing, then per chunk of tokens a layout (two
// sets, so that the next chunk's can be built on the aux stream while the current one is
// in use), the routed FFN and the combine; optional shared-expert rows per set.
moe_problem shared_problem(const moe_problem& p, int rows, int shared_I) {
  moe_problem ps = p;
  ps.T = rows;
  ps.E = 1;
  ps.k = 1;
  ps.I = shared_I;
  ps.capacity = 0;
  return ps;
}

int chunked_check(const moe_problem* p, int chunk_tokens, int shared_I) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (chunk_tokens < 1 || shared_I < 0) return MOE_ERR_INVALID_ARG;
  if (shared_I > 0) {
    moe_problem ps = shared_problem(*p, std::min(chunk_tokens, p->T), shared_I);
    if ((st = moe_problem_check(&ps)) != MOE_OK) return st;
  }
  return MOE_OK;
}

struct ChunkSet {
  int32_t *counts, *offsets, *row_token, *slot_to_row, *s_off;
  RankScratch rank;
  FfnScratch s_ffn;  // shared expert's intermediate (and quantised rows)
  void* ys;          // shared expert's output rows
};
struct ChunkScratch {
  int32_t* ids;
  float* w;
  uint8_t* keep;
  RankScratch rank;  // capacity over all T
  ChunkSet set[2];
  FfnScratch ffn;    // routed intermediate of one chunk
  void* yp;
};
ChunkScratch carve_chunked(Carve& c, const moe_problem& p, int chunk_tokens, int shared_I) {
  const int tc = std::min(chunk_tokens, p.T);
  const size_t tk = (size_t)p.T * p.k, ck = (size_t)tc * p.k;
  const size_t eb = elem_bytes(p.act_dtype);
  moe_problem pc = p;
  pc.T = tc;
  ChunkScratch S{};
  S.ids = c.take<int32_t>(tk);
  S.w = c.take<float>(tk);
  S.keep = c.take<uint8_t>(tk);
  S.rank = p.capacity > 0 ? carve_rank(c, p, true) : RankScratch{};
  for (int i = 0; i < 2; ++i) {
    ChunkSet& L = S.set[i];
    L.counts = c.take<int32_t>(p.E);
    L.offsets = c.take<int32_t>((size_t)p.E + 1);
    L.row_token = c.take<int32_t>(ck);
    L.slot_to_row = c.take<int32_t>(ck);
    L.rank = carve_rank(c, pc, false);
    if (shared_I > 0) {
      L.s_off = c.take<int32_t>(2);
      L.s_ffn = carve_ffn(c, shared_problem(p, tc, shared_I));
      L.ys = c.take<char>((size_t)tc * p.H * eb);
    }
  }
  S.ffn = carve_ffn(c, pc);
  S.yp = c.take<char>(ck * p.H * eb);
  return S;
}

struct LayerScratch {
  int32_t *ids, *counts, *offsets, *row_token, *slot_to_row;
  int32_t* claims;  // the prefill GEMMs' work-item counters (zeroed by the layout)
  float* w;
  uint8_t* keep;
  void* yp;
  RankScratch rank;
  FfnScratch ffn;
};
LayerScratch carve_layer(Carve& c, const moe_problem& p) {
  const size_t tk = (size_t)p.T * p.k;
  const size_t eb = elem_bytes(p.act_dtype);
  LayerScratch L{};
  L.ids = c.take<int32_t>(tk);
  L.w = c.take<float>(tk);
  L.keep = c.take<uint8_t>(tk);
  L.counts = c.take<int32_t>(p.E);
  L.offsets = c.take<int32_t>((size_t)p.E + 1);
  L.row_token = c.take<int32_t>(tk);
  L.slot_to_row = c.take<int32_t>(tk);
  L.claims = c.take<int32_t>(kClaimInts);
  L.yp = c.take<char>(tk * p.H * eb);
  L.rank = carve_rank(c, p, p.capacity > 0);
  L.ffn = carve_ffn(c, p);
  return L;
}

// Routing scratch: the capacity pipeline's, only with a cap.
RankScratch carve_route(Carve& c, const moe_problem& p) {
  return p.capacity > 0 ? carve_rank(c, p, true) : RankScratch{};
}

// Router scratch: the split-K partial logit planes, then the routing scratch.
struct RouterScratch {
  float* part;
  RankScratch rank;
};
RouterScratch carve_router(Carve& c, const moe_problem& p) {
  RouterScratch r{};
  r.part = c.take<float>((size_t)router_plan(p).split * p.T * p.E);
  r.rank = carve_route(c, p);
  return r;
}

// ---- backward pass scratch: bf16 row buffers of the layout, their padded transposes, the
// router's parts.
bool backward_supported(const moe_problem& p, bool router) {
  return p.act_dtype == MOE_BF16 && p.w_dtype == MOE_BF16 && p.H % 128 == 0 &&
         p.H <= 8192 && (!router || p.E % 64 == 0);
}
bool router_bwd_ok(const moe_problem& p) { return p.E % 64 == 0; }

struct BwdScratch {
  float* dw;       // d topk_w when the caller does not want it
  void *dyp, *da, *gu, *dgu, *dxp, *yp;
  FfnScratch ffn;  // the yp recompute's intermediate
  int32_t* poff;
  int64_t npad;    // row stride of the transposes
  void *xT, *aT, *dypT, *dguT;
  // router
  void *dl16, *dxr, *wr_packed, *dlT, *xTf;
  int32_t *roff, *rpoff;
  int64_t tpad;
};
BwdScratch carve_backward(Carve& c, const moe_problem& p, bool router) {
  const size_t tk = (size_t)p.T * p.k;
  BwdScratch B{};
  B.npad = (int64_t)((tk + 64 * (size_t)p.E + 63) & ~(size_t)63);  // rows padded per expert
  B.dw = c.take<float>(tk);
  B.dyp = c.take<uint16_t>(tk * p.H);
  B.da = c.take<uint16_t>(tk * p.I);
  B.gu = c.take<uint16_t>(tk * 2 * p.I);
  B.dgu = c.take<uint16_t>(tk * 2 * p.I);
  B.dxp = c.take<uint16_t>(tk * p.H);
  B.yp = c.take<uint16_t>(tk * p.H);
  B.ffn = carve_ffn(c, p);
  B.poff = c.take<int32_t>((size_t)p.E + 1);
  B.xT = c.take<uint16_t>((size_t)p.H * B.npad);
  B.aT = c.take<uint16_t>((size_t)p.I * B.npad);
  B.dypT = c.take<uint16_t>((size_t)p.H * B.npad);
  B.dguT = c.take<uint16_t>((size_t)2 * p.I * B.npad);
  if (router) {
    B.tpad = (int64_t)(((size_t)p.T + 63) & ~(size_t)63);
    B.dl16 = c.take<uint16_t>((size_t)p.T * p.E);
    B.dxr = c.take<uint16_t>((size_t)p.T * p.H);
    B.wr_packed = c.take<uint16_t>((size_t)p.E * p.H);
    B.roff = c.take<int32_t>(2);
    B.rpoff = c.take<int32_t>(2);
    B.dlT = c.take<uint16_t>((size_t)p.E * B.tpad);
    B.xTf = c.take<uint16_t>((size_t)p.H * B.tpad);
  }
  return B;
}

// Every entry point carves its workspace with the same function that sizes it here.
size_t ws_bytes_of(const moe_problem& p, int op) {
  Carve c(nullptr);
  switch (op) {
    case MOE_OP_ROUTE:
      carve_route(c, p);
      break;
    case MOE_OP_ROUTER:
      if (!router_supported(p)) return 0;
      carve_router(c, p);
      break;
    case MOE_OP_DISPATCH:
      carve_rank(c, p, false);
      break;
    case MOE_OP_BACKWARD:
      if (!backward_supported(p, false)) return 0;
      carve_backward(c, p, router_bwd_ok(p));
      break;
    case MOE_OP_FFN:
      carve_ffn(c, p);
      break;
    case MOE_OP_COMBINE:
      break;
    case MOE_OP_LAYER:
      carve_layer(c, p);
      break;
    default:
      return 0;
  }
  return c.used;
}

int check_ws(const moe_problem* p, int op, const void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_of(*p, op);
  if (need == 0) return MOE_OK;
  if (!ws) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255) != 0) return MOE_ERR_INVALID_ARG;
  return ws_bytes < need ? MOE_ERR_WORKSPACE : MOE_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ---- aliasing.  A call's outputs (the workspace included) must not overlap its inputs or
// each other; inputs may share memory.  Byte ranges come from the problem's shapes (row
// buffers hold T*k rows); NULL or empty ranges overlap nothing.
struct Span {
  const void* p;
  size_t n;
};
bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}
bool aliased(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
  for (auto o = outs.begin(); o != outs.end(); ++o) {
    for (const Span& i : ins)
      if (overlap(*o, i)) return true;
    for (auto o2 = o + 1; o2 != outs.end(); ++o2)
      if (overlap(*o, *o2)) return true;
  }
  return false;
}
// Sizes of the shaped buffers of problem p.
size_t tk_of(const moe_problem& p) { return (size_t)p.T * p.k; }
size_t act_rows(const moe_problem& p, size_t rows, size_t cols) {
  return rows * cols * elem_bytes(p.act_dtype);
}
size_t a_bytes(const moe_problem& p) {  // the FFN intermediate [T*k, I]
  return is_fp8(p) ? q_rows_bytes(tk_of(p), p.I) : act_rows(p, tk_of(p), p.I);
}
size_t natural_w_bytes(const moe_problem& p) {  // one natural weight set [E, H, I]
  return (size_t)p.E * p.H * p.I * (p.w_dtype == MOE_F32 ? 4 : 2);
}

// Capacity after the selection: candidate layout + radix select (no-op without a cap).
hipError_t run_capacity(const moe_problem& p, int32_t* ids, float* w, uint8_t* keep,
                        const RankScratch& r, hipStream_t s) {
  hipError_t err = hipSuccess;
  if (p.capacity <= 0) return err;
  if ((err = launch_layout(p, ids, nullptr, r.chunk_hist, r.chunk_base, r.cand_counts,
                           r.cand_offsets, nullptr, nullptr, r.cand_slot, s)) != hipSuccess)
    return err;
  return launch_capacity_select(p, r.cand_counts, r.cand_offsets, r.cand_slot, w, keep, s);
}

// The routing pipeline: top-k (group-limited if asked), then the capacity.
hipError_t run_route(const moe_problem& p, const float* logits, int n_group, int topk_group,
                     int32_t* ids, float* w, uint8_t* keep, const RankScratch& r,
                     hipStream_t s) {
  hipError_t err = launch_route(p, logits, n_group, topk_group, ids, w, keep, s);
  return err != hipSuccess ? err : run_capacity(p, ids, w, keep, r, s);
}

// 1 <= topk_group <= n_group <= 64, n_group divides E, k fits in the taken groups.
bool groups_ok(const moe_problem& p, int n_group, int topk_group) {
  return n_group >= 1 && n_group <= 64 && p.E % n_group == 0 && topk_group >= 1 &&
         topk_group <= n_group && (int64_t)topk_group * (p.E / n_group) >= p.k;
}

hipError_t run_dispatch(const moe_problem& p, const void* x, const int32_t* ids,
                        const uint8_t* keep, int32_t* counts, int32_t* offsets,
                        int32_t* row_token, int32_t* slot_to_row, void* xp,
                        const RankScratch& r, hipStream_t s, int32_t* zero_claims = nullptr) {
  hipError_t err = hipSuccess;
#ifdef MOE_DEBUG_CHECKS
  err = launch_check_ids(p, ids, s);  // the ids may be the caller's
  if (err != hipSuccess) return err;
#endif
  err = launch_layout(p, ids, keep, r.chunk_hist, r.chunk_base, counts, offsets, row_token,
                      slot_to_row, nullptr, s, zero_claims);
  if (err == hipSuccess && xp) err = launch_gather(p, x, slot_to_row, xp, s);
  return err;
}

// Gate/up over the layout: rows xs[r], or token rows xs[row_token[r]] if row_token != NULL.
// FP8: the input rows (T token rows, or T*k rows of xp) are quantised into f.xq first.
// decode: which bf16 kernel family (ffn_use_decode of the problem the rows belong to).
// gu (bf16 only): also store the pre-activations g|u.
hipError_t run_gate_up(const moe_problem& p, const void* xs, const int32_t* row_token,
                       const int32_t* offsets, const void* pgu, void* a, const FfnScratch& f,
                       bool decode, hipStream_t s, void* gu = nullptr, int* claim = nullptr) {
  if (is_fp8(p)) {
    const size_t tk = (size_t)p.T * p.k;
    const size_t rows = row_token ? (size_t)p.T : tk;
    uint8_t* xq = static_cast<uint8_t*>(f.xq);
    uint8_t* xsc = q_scales(f.xq, tk, p.H);
    // layout rows: only the N = offsets[E] filled ones
    hipError_t err = launch_quant_rows(xs, (int64_t)rows, p.H, row_token ? nullptr : offsets + p.E,
                                       xq, xsc, s);
    if (err != hipSuccess) return err;
    return launch_gate_up_fp8(p, xq, xsc, row_token, offsets, pgu, static_cast<uint8_t*>(a),
                              q_scales(a, tk, p.I), s);
  }
  if (p.act_dtype == MOE_F32) {
    const size_t n = (size_t)p.E * p.H * p.I;
    return launch_gate_up_f32(p, (const float*)xs, row_token, offsets, (const float*)pgu,
                              (const float*)pgu + n, (float*)a, s);
  }
  return launch_gate_up_bf16(p, xs, row_token, offsets, pgu, a, gu, decode, s, claim);
}

hipError_t run_down(const moe_problem& p, const void* a, const int32_t* offsets,
                    const void* pd, void* yp, bool decode, hipStream_t s, int* claim = nullptr) {
  if (is_fp8(p)) {
    const size_t tk = (size_t)p.T * p.k;
    return launch_down_fp8(p, static_cast<const uint8_t*>(a),
                           q_scales(const_cast<void*>(a), tk, p.I), offsets, pd, yp, s);
  }
  if (p.act_dtype == MOE_F32)
    return launch_down_f32(p, (const float*)a, offsets, (const float*)pd, (float*)yp, s);
  return launch_down_bf16(p, a, offsets, pd, yp, decode, s, claim);
}

// ---- the no-allocation layer (moe_layer_static): moe_layer's workspace in a file-scope
// device array, its address looked up once per device (the array's name is only a host-side
// stand-in: kernels must be given the device address).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (NULL on failure).
void* static_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported problem";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int moe_problem_check(const moe_problem* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (p->T < 1 || p->H < 1 || p->E < 1 || p->k < 1 || p->I < 1) return MOE_ERR_INVALID_ARG;
  if (p->k > p->E) return MOE_ERR_INVALID_ARG;
  if ((p->act_dtype != MOE_F32 && p->act_dtype != MOE_BF16) ||
      (p->w_dtype != MOE_F32 && p->w_dtype != MOE_BF16 && p->w_dtype != MOE_FP8))
    return MOE_ERR_INVALID_ARG;
  if (p->renormalize != 0 && p->renormalize != 1) return MOE_ERR_INVALID_ARG;
  if (p->E > kMaxE || p->k > 32) return MOE_ERR_UNSUPPORTED;
  if (p->w_dtype == MOE_FP8) {
    // FP8 weights take bf16 activations; a stage of the FP8 GEMM is 128 elements of K
    if (p->act_dtype != MOE_BF16 || p->H % 128 || p->I % 128) return MOE_ERR_UNSUPPORTED;
  } else if (p->act_dtype != p->w_dtype) {
    return MOE_ERR_UNSUPPORTED;
  }
  const int mult = p->act_dtype == MOE_BF16 ? 64 : 8;
  if (p->H % mult || p->I % mult) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)p->T * p->k >= ((int64_t)1 << 31) - 2 * (int64_t)kPrefillBM * 1024)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_workspace_bytes(const moe_problem* p, int op) {
  if (moe_problem_check(p) != MOE_OK) return 0;
  return ws_bytes_of(*p, op);
}

size_t moe_packed_bytes(const moe_problem* p, int which) {
  if (moe_problem_check(p) != MOE_OK) return 0;
  if (p->w_dtype == MOE_FP8) {
    if (which == MOE_W_GATE_UP)
      return align256(fp8_packed_code_bytes(p->E, p->H, p->I, 2)) +
             fp8_packed_scale_bytes(p->E, p->H, p->I, 2);
    if (which == MOE_W_DOWN)
      return align256(fp8_packed_code_bytes(p->E, p->I, p->H, 1)) +
             fp8_packed_scale_bytes(p->E, p->I, p->H, 1);
    return 0;
  }
  const size_t n = (size_t)p->E * p->H * p->I * elem_bytes(p->w_dtype);
  if (which == MOE_W_GATE_UP) return 2 * n;
  if (which == MOE_W_DOWN) return n;
  return 0;
}

int moe_pack_weights(const moe_problem* p, const void* w_gate, const void* w_up,
                     const void* w_down, void* packed_gate_up, void* packed_down,
                     void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!w_gate || !w_up || !w_down || !packed_gate_up || !packed_down)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(packed_gate_up) || !aligned16(packed_down)) return MOE_ERR_INVALID_ARG;
  {
    const size_t nw = natural_w_bytes(*p);
    if (aliased({{packed_gate_up, moe_packed_bytes(p, MOE_W_GATE_UP)},
                 {packed_down, moe_packed_bytes(p, MOE_W_DOWN)}},
                {{w_gate, nw}, {w_up, nw}, {w_down, nw}}))
      return MOE_ERR_INVALID_ARG;
  }
  if (p->w_dtype == MOE_FP8)
    return status_of(launch_pack_fp8(*p, w_gate, w_up, w_down, packed_gate_up, packed_down,
                                     as_stream(stream)));
  return status_of(
      launch_pack(*p, w_gate, w_up, w_down, packed_gate_up, packed_down, as_stream(stream)));
}

int moe_route(const moe_problem* p, const float* logits, int32_t* topk_ids, float* topk_w,
              uint8_t* keep, void* ws, size_t ws_bytes, void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!logits || !topk_ids || !topk_w || !keep) return MOE_ERR_INVALID_ARG;
  if (aliased({{topk_ids, tk_of(*p) * 4}, {topk_w, tk_of(*p) * 4}, {keep, tk_of(*p)},
               {ws, ws_bytes}},
              {{logits, (size_t)p->T * p->E * 4}}))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(p, MOE_OP_ROUTE, ws, ws_bytes)) != MOE_OK) return st;
  Carve c(ws);
  RankScratch r = carve_route(c, *p);
  if (c.used > ws_bytes) return MOE_ERR_WORKSPACE;  // (sized by the same carve)
  return status_of(run_route(*p, logits, 1, 1, topk_ids, topk_w, keep, r, as_stream(stream)));
}

int moe_route_grouped(const moe_problem* p, const float* logits, int32_t n_group,
                      int32_t topk_group, int32_t* topk_ids, float* topk_w, uint8_t* keep,
                      void* ws, size_t ws_bytes, void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!logits || !topk_ids || !topk_w || !keep || !groups_ok(*p, n_group, topk_group))
    return MOE_ERR_INVALID_ARG;
  if (aliased({{topk_ids, tk_of(*p) * 4}, {topk_w, tk_of(*p) * 4}, {keep, tk_of(*p)},
               {ws, ws_bytes}},
              {{logits, (size_t)p->T * p->E * 4}}))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(p, MOE_OP_ROUTE, ws, ws_bytes)) != MOE_OK) return st;
  Carve c(ws);
  RankScratch r = carve_route(c, *p);
  if (c.used > ws_bytes) return MOE_ERR_WORKSPACE;  // (sized by the same carve)
  return status_of(run_route(*p, logits, n_group, topk_group, topk_ids, topk_w, keep, r,
                             as_stream(stream)));
}

int moe_router(const moe_problem* p, const void* x, const void* w_router, int32_t n_group,
               int32_t topk_group, float* logits, int32_t* topk_ids, float* topk_w,
               uint8_t* keep, void* ws, size_t ws_bytes, void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !topk_ids || !topk_w || !keep || !groups_ok(*p, n_group, topk_group))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID_ARG;
  if (!router_supported(*p)) return MOE_ERR_UNSUPPORTED;
  if (aliased({{logits, (size_t)p->T * p->E * 4}, {topk_ids, tk_of(*p) * 4},
               {topk_w, tk_of(*p) * 4}, {keep, tk_of(*p)}, {ws, ws_bytes}},
              {{x, (size_t)p->T * p->H * 2}, {w_router, (size_t)p->E * p->H * 2}}))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(p, MOE_OP_ROUTER, ws, ws_bytes)) != MOE_OK) return st;
  Carve c(ws);
  RouterScratch r = carve_router(c, *p);
  if (c.used > ws_bytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  hipError_t err = launch_router(*p, x, w_router, n_group, topk_group, r.part, logits, topk_ids,
                                 topk_w, keep, s);
  if (err == hipSuccess) err = run_capacity(*p, topk_ids, topk_w, keep, r.rank, s);
  return status_of(err);
}

int moe_dispatch(const moe_problem* p, const void* x, const int32_t* topk_ids,
                 const uint8_t* keep, int32_t* counts, int32_t* offsets, int32_t* row_token,
                 int32_t* slot_to_row, void* xp, void* ws, size_t ws_bytes, void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!x || !topk_ids || !counts || !offsets || !row_token || !slot_to_row)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || (xp && !aligned16(xp))) return MOE_ERR_INVALID_ARG;
  if (aliased({{counts, (size_t)p->E * 4}, {offsets, ((size_t)p->E + 1) * 4},
               {row_token, tk_of(*p) * 4}, {slot_to_row, tk_of(*p) * 4},
               {xp, act_rows(*p, tk_of(*p), p->H)}, {ws, ws_bytes}},
              {{x, act_rows(*p, p->T, p->H)}, {topk_ids, tk_of(*p) * 4}, {keep, tk_of(*p)}}))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(p, MOE_OP_DISPATCH, ws, ws_bytes)) != MOE_OK) return st;
  Carve c(ws);
  RankScratch r = carve_rank(c, *p, false);
  if (c.used > ws_bytes) return MOE_ERR_WORKSPACE;  // (sized by the same carve)
  return status_of(run_dispatch(*p, x, topk_ids, keep, counts, offsets, row_token, slot_to_row,
                                xp, r, as_stream(stream)));
}

int moe_expert_gate_up(const moe_problem* p, const void* xp, const int32_t* offsets,
                       const void* packed_gate_up, void* a, void* ws, size_t ws_bytes,
                       void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!xp || !offsets || !packed_gate_up || !a) return MOE_ERR_INVALID_ARG;
  if (!aligned16(xp) || !aligned16(packed_gate_up) || !aligned16(a)) return MOE_ERR_INVALID_ARG;
  if (aliased({{a, a_bytes(*p)}, {is_fp8(*p) ? ws : nullptr, ws_bytes}},
              {{xp, act_rows(*p, tk_of(*p), p->H)}, {offsets, ((size_t)p->E + 1) * 4},
               {packed_gate_up, moe_packed_bytes(p, MOE_W_GATE_UP)}}))
    return MOE_ERR_INVALID_ARG;
  FfnScratch f{};
  if (is_fp8(*p)) {  // the quantised input rows live in the workspace
    if ((st = check_ws(p, MOE_OP_FFN, ws, ws_bytes)) != MOE_OK) return st;
    Carve c(ws);
    f = carve_ffn(c, *p);
    if (c.used > ws_bytes) return MOE_ERR_WORKSPACE;  // (sized by the same carve)
  }
  return status_of(
      run_gate_up(*p, xp, nullptr, offsets, packed_gate_up, a, f,
                  ffn_use_decode(*p), as_stream(stream)));
}

int moe_expert_gate_up_gather(const moe_problem* p, const void* x, const int32_t* row_token,
                              const int32_t* offsets, const void* packed_gate_up, void* a,
                              void* ws, size_t ws_bytes, void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!x || !row_token || !offsets || !packed_gate_up || !a) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(packed_gate_up) || !aligned16(a)) return MOE_ERR_INVALID_ARG;
  if (aliased({{a, a_bytes(*p)}, {is_fp8(*p) ? ws : nullptr, ws_bytes}},
              {{x, act_rows(*p, p->T, p->H)}, {row_token, tk_of(*p) * 4},
               {offsets, ((size_t)p->E + 1) * 4},
               {packed_gate_up, moe_packed_bytes(p, MOE_W_GATE_UP)}}))
    return MOE_ERR_INVALID_ARG;
  FfnScratch f{};
  if (is_fp8(*p)) {
    if ((st = check_ws(p, MOE_OP_FFN, ws, ws_bytes)) != MOE_OK) return st;
    Carve c(ws);
    f = carve_ffn(c, *p);
    if (c.used > ws_bytes) return MOE_ERR_WORKSPACE;  // (sized by the same carve)
  }
  return status_of(
      run_gate_up(*p, x, row_token, offsets, packed_gate_up, a, f,
                  ffn_use_decode(*p), as_stream(stream)));
}

int moe_expert_gate_up_gather_gu(const moe_problem* p, const void* x, const int32_t* row_token,
                                 const int32_t* offsets, const void* packed_gate_up, void* a,
                                 void* gu, void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!backward_supported(*p, false)) return MOE_ERR_UNSUPPORTED;
  if (!x || !row_token || !offsets || !packed_gate_up || !a || !gu) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(packed_gate_up) || !aligned16(a) || !aligned16(gu))
    return MOE_ERR_INVALID_ARG;
  if (aliased({{a, a_bytes(*p)}, {gu, tk_of(*p) * 2 * p->I * 2}},
              {{x, act_rows(*p, p->T, p->H)}, {row_token, tk_of(*p) * 4},
               {offsets, ((size_t)p->E + 1) * 4},
               {packed_gate_up, moe_packed_bytes(p, MOE_W_GATE_UP)}}))
    return MOE_ERR_INVALID_ARG;
  return status_of(run_gate_up(*p, x, row_token, offsets, packed_gate_up, a, FfnScratch{},
                               ffn_use_decode(*p), as_stream(stream), gu));
}

int moe_quantize_fp8(const void* x, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                     void* stream) {
  if (rows < 0 || cols <= 0 || cols % 32) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales || !aligned16(x) || !aligned16(codes)) return MOE_ERR_INVALID_ARG;
  if (aliased({{codes, (size_t)rows * cols}, {scales, (size_t)rows * (cols / 32)}},
              {{x, (size_t)rows * cols * 2}}))
    return MOE_ERR_INVALID_ARG;
  return status_of(launch_quant_rows(x, rows, cols, nullptr, codes, scales, as_stream(stream)));
}

int moe_expert_down(const moe_problem* p, const void* a, const int32_t* offsets,
                    const void* packed_down, void* yp, void* ws, size_t ws_bytes,
                    void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!a || !offsets || !packed_down || !yp) return MOE_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(packed_down) || !aligned16(yp)) return MOE_ERR_INVALID_ARG;
  if (aliased({{yp, act_rows(*p, tk_of(*p), p->H)}},
              {{a, a_bytes(*p)}, {offsets, ((size_t)p->E + 1) * 4},
               {packed_down, moe_packed_bytes(p, MOE_W_DOWN)}}))
    return MOE_ERR_INVALID_ARG;
  (void)ws;
  (void)ws_bytes;
  return status_of(
      run_down(*p, a, offsets, packed_down, yp, ffn_use_decode(*p), as_stream(stream)));
}

int moe_expert_ffn(const moe_problem* p, const void* xp, const int32_t* offsets,
                   const void* packed_gate_up, const void* packed_down, void* yp, void* ws,
                   size_t ws_bytes, void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!xp || !offsets || !packed_gate_up || !packed_down || !yp) return MOE_ERR_INVALID_ARG;
  if (!aligned16(xp) || !aligned16(packed_gate_up) || !aligned16(packed_down) ||
      !aligned16(yp))
    return MOE_ERR_INVALID_ARG;
  if (aliased({{yp, act_rows(*p, tk_of(*p), p->H)}, {ws, ws_bytes}},
              {{xp, act_rows(*p, tk_of(*p), p->H)}, {offsets, ((size_t)p->E + 1) * 4},
               {packed_gate_up, moe_packed_bytes(p, MOE_W_GATE_UP)},
               {packed_down, moe_packed_bytes(p, MOE_W_DOWN)}}))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(p, MOE_OP_FFN, ws, ws_bytes)) != MOE_OK) return st;
  Carve c(ws);
  FfnScratch f = carve_ffn(c, *p);
  if (c.used > ws_bytes) return MOE_ERR_WORKSPACE;  // (sized by the same carve)
  hipStream_t s = as_stream(stream);
  const bool dec = ffn_use_decode(*p);
  hipError_t err = run_gate_up(*p, xp, nullptr, offsets, packed_gate_up, f.a, f, dec, s);
  if (err == hipSuccess) err = run_down(*p, f.a, offsets, packed_down, yp, dec, s);
  return status_of(err);
}

int moe_combine(const moe_problem* p, const void* yp, const float* topk_w,
                const int32_t* slot_to_row, void* y, void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!yp || !topk_w || !slot_to_row || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(yp) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  if (aliased({{y, act_rows(*p, p->T, p->H)}},
              {{yp, act_rows(*p, tk_of(*p), p->H)}, {topk_w, tk_of(*p) * 4},
               {slot_to_row, tk_of(*p) * 4}}))
    return MOE_ERR_INVALID_ARG;
  return status_of(launch_combine(*p, yp, topk_w, slot_to_row, nullptr, y, as_stream(stream)));
}

int moe_layer(const moe_problem* p, const void* x, const float* logits,
              const void* packed_gate_up, const void* packed_down, void* y, int32_t* topk_ids,
              float* topk_w, uint8_t* keep, int32_t* counts, int32_t* offsets,
              int32_t* row_token, int32_t* slot_to_row, void* ws, size_t ws_bytes,
              void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!x || !logits || !packed_gate_up || !packed_down || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(packed_gate_up) || !aligned16(packed_down))
    return MOE_ERR_INVALID_ARG;
  {
    const size_t tk = tk_of(*p);
    if (aliased({{y, act_rows(*p, p->T, p->H)}, {topk_ids, tk * 4}, {topk_w, tk * 4},
                 {keep, tk}, {counts, (size_t)p->E * 4}, {offsets, ((size_t)p->E + 1) * 4},
                 {row_token, tk * 4}, {slot_to_row, tk * 4}, {ws, ws_bytes}},
                {{x, act_rows(*p, p->T, p->H)}, {logits, (size_t)p->T * p->E * 4},
                 {packed_gate_up, moe_packed_bytes(p, MOE_W_GATE_UP)},
                 {packed_down, moe_packed_bytes(p, MOE_W_DOWN)}}))
      return MOE_ERR_INVALID_ARG;
  }
  if ((st = check_ws(p, MOE_OP_LAYER, ws, ws_bytes)) != MOE_OK) return st;
  Carve c(ws);
  LayerScratch L = carve_layer(c, *p);
  if (c.used > ws_bytes) return MOE_ERR_WORKSPACE;  // (sized by the same carve)
  if (!topk_ids) topk_ids = L.ids;
  if (!topk_w) topk_w = L.w;
  if (!keep) keep = L.keep;
  if (!counts) counts = L.counts;
  if (!offsets) offsets = L.offsets;
  if (!row_token) row_token = L.row_token;
  if (!slot_to_row) slot_to_row = L.slot_to_row;
  hipStream_t s = as_stream(stream);
  hipError_t err = run_route(*p, logits, 1, 1, topk_ids, topk_w, keep, L.rank, s);
  // dispatch builds the layout only: gate/up reads the token rows through row_token
  if (err == hipSuccess)
    err = run_dispatch(*p, x, topk_ids, p->capacity > 0 ? keep : nullptr, counts, offsets,
                       row_token, slot_to_row, nullptr, L.rank, s, L.claims);
  if (err == hipSuccess)
    err = run_gate_up(*p, x, row_token, offsets, packed_gate_up, L.ffn.a, L.ffn,
                      ffn_use_decode(*p), s, nullptr, L.claims);
  if (err == hipSuccess)
    err = run_down(*p, L.ffn.a, offsets, packed_down, L.yp, ffn_use_decode(*p), s,
                   L.claims + kClaimInts / 2);
  if (err == hipSuccess) err = launch_combine(*p, L.yp, topk_w, slot_to_row, nullptr, y, s);
  return status_of(err);
}

size_t moe_layer_static_max_bytes(void) { return kStaticScratchBytes; }

int moe_layer_static(const moe_problem* p, const void* x, const float* logits,
                     const void* packed_gate_up, const void* packed_down, void* y,
                     int32_t* topk_ids, float* topk_w, uint8_t* keep, int32_t* counts,
                     int32_t* offsets, int32_t* row_token, int32_t* slot_to_row, void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  const size_t need = ws_bytes_of(*p, MOE_OP_LAYER);
  if (need > kStaticScratchBytes) return MOE_ERR_WORKSPACE;
  void* ws = static_scratch();
  if (!ws) return MOE_ERR_HIP;
  // every kernel of the layer writes what it later reads: nothing in the scratch needs
  // clearing between calls
  return moe_layer(p, x, logits, packed_gate_up, packed_down, y, topk_ids, topk_w, keep, counts,
                   offsets, row_token, slot_to_row, ws, kStaticScratchBytes, stream);
}

int moe_pack_weights_backward(const moe_problem* p, const void* w_gate, const void* w_up,
                              const void* w_down, void* packed_bwd_gate_up,
                              void* packed_bwd_down, void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!backward_supported(*p, false)) return MOE_ERR_UNSUPPORTED;
  if (!w_gate || !w_up || !w_down || !packed_bwd_gate_up || !packed_bwd_down)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(packed_bwd_gate_up) || !aligned16(packed_bwd_down)) return MOE_ERR_INVALID_ARG;
  {
    const size_t nw = natural_w_bytes(*p);
    if (aliased({{packed_bwd_gate_up, moe_packed_bytes(p, MOE_W_GATE_UP)},
                 {packed_bwd_down, moe_packed_bytes(p, MOE_W_DOWN)}},
                {{w_gate, nw}, {w_up, nw}, {w_down, nw}}))
      return MOE_ERR_INVALID_ARG;
  }
  return status_of(launch_pack_backward(*p, w_gate, w_up, w_down, packed_bwd_gate_up,
                                        packed_bwd_down, as_stream(stream)));
}

int moe_layer_backward(const moe_problem* p, const void* x, const float* logits,
                       const void* w_router, const void* packed_gate_up,
                       const void* packed_down, const void* packed_bwd_gate_up,
                       const void* packed_bwd_down, const moe_saved_routing* saved,
                       const void* yp, const void* gu, const void* dy, const moe_grads* grads,
                       void* ws, size_t ws_bytes, void* stream) {
  int st = moe_problem_check(p);
  if (st != MOE_OK) return st;
  if (!backward_supported(*p, w_router != nullptr)) return MOE_ERR_UNSUPPORTED;
  if (!x || !packed_gate_up || !packed_bwd_gate_up || !packed_bwd_down || !saved || !dy ||
      !grads)
    return MOE_ERR_INVALID_ARG;
  if (!saved->topk_ids || !saved->topk_w || !saved->offsets || !saved->row_token ||
      !saved->slot_to_row)
    return MOE_ERR_INVALID_ARG;
  if (!grads->dx || !grads->dw_gate || !grads->dw_up || !grads->dw_down || !grads->dlogits ||
      (w_router && !grads->dw_router) || (!p->renormalize && !logits) ||
      (!yp && !packed_down))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(grads->dx) || (yp && !aligned16(yp)) ||
      (gu && !aligned16(gu)) || (w_router && !aligned16(w_router)))
    return MOE_ERR_INVALID_ARG;
  {
    const size_t tk = tk_of(*p), TH2 = (size_t)p->T * p->H * 2;
    const size_t ew = (size_t)p->E * p->H * p->I * 4;
    const moe_saved_routing& R = *saved;
    if (aliased({{grads->dx, TH2}, {grads->dw_gate, ew}, {grads->dw_up, ew},
                 {grads->dw_down, ew}, {grads->dlogits, (size_t)p->T * p->E * 4},
                 {grads->dtopk_w, tk * 4},
                 {w_router ? grads->dw_router : nullptr, (size_t)p->E * p->H * 4},
                 {ws, ws_bytes}},
                {{x, TH2}, {logits, (size_t)p->T * p->E * 4},
                 {w_router, (size_t)p->E * p->H * 2},
                 {packed_gate_up, moe_packed_bytes(p, MOE_W_GATE_UP)},
                 {packed_down, moe_packed_bytes(p, MOE_W_DOWN)},
                 {packed_bwd_gate_up, moe_packed_bytes(p, MOE_W_GATE_UP)},
                 {packed_bwd_down, moe_packed_bytes(p, MOE_W_DOWN)}, {R.topk_ids, tk * 4},
                 {R.topk_w, tk * 4}, {R.offsets, ((size_t)p->E + 1) * 4},
                 {R.row_token, tk * 4}, {R.slot_to_row, tk * 4}, {yp, tk * p->H * 2},
                 {gu, tk * 2 * p->I * 2}, {dy, TH2}}))
      return MOE_ERR_INVALID_ARG;
  }
  if ((st = check_ws(p, MOE_OP_BACKWARD, ws, ws_bytes)) != MOE_OK) return st;
  Carve c(ws);
  BwdScratch B = carve_backward(c, *p, router_bwd_ok(*p));
  if (c.used > ws_bytes) return MOE_ERR_WORKSPACE;  // (sized by the same carve)
  hipStream_t s = as_stream(stream);
  const moe_saved_routing& R = *saved;
  const bool dec = ffn_use_decode(*p);
  const int H = p->H, I = p->I, E = p->E;
  float* dw = grads->dtopk_w ? grads->dtopk_w : B.dw;
  hipError_t err = hipSuccess;
#ifdef MOE_DEBUG_CHECKS
  err = launch_check_ids(*p, R.topk_ids, s);  // the saved routing comes from the caller
#endif
  // the forward's expert outputs, if not saved
  if (!yp) {
    err = run_gate_up(*p, x, R.row_token, R.offsets, packed_gate_up, B.ffn.a, B.ffn, dec, s);
    if (err == hipSuccess) err = run_down(*p, B.ffn.a, R.offsets, packed_down, B.yp, dec, s);
    yp = B.yp;
  }
  // combine and routing backward
  if (err == hipSuccess) err = launch_combine_bwd(*p, dy, yp, R.topk_w, R.slot_to_row, B.dyp, dw, s);
  if (err == hipSuccess) err = launch_route_bwd(*p, logits, R.topk_ids, R.topk_w, dw, grads->dlogits, s);
  // data gradients: da = dyp W_down^T; g|u (saved, or recomputed); SwiGLU backward;
  // dxp = dgu [Wg|Wu]^T
  if (err == hipSuccess)
    err = launch_gemm_bf16(E, B.dyp, nullptr, R.offsets, packed_bwd_down, B.da, H, I, dec, s);
  if (err == hipSuccess && !gu) {
    err = launch_gemm_bf16(E, x, R.row_token, R.offsets, packed_gate_up, B.gu, H, 2 * I, dec, s);
    gu = B.gu;
  }
  if (err == hipSuccess) err = launch_pad_offsets(R.offsets, E, 64, B.poff, s);
  if (err == hipSuccess)
    err = launch_swiglu_bwd(*p, gu, B.da, R.offsets, B.poff, B.npad, B.dgu, B.dguT, B.aT, s);
  if (err == hipSuccess)
    err = launch_gemm_bf16(E, B.dgu, nullptr, R.offsets, packed_bwd_gate_up, B.dxp, 2 * I, H,
                           dec, s);
  // the router's path: dx_r = dlogits W_r (added in the sum below), dW_r = dlogits^T x
  const void* dxr = nullptr;
  if (w_router && err == hipSuccess) {
    err = launch_f32_to_bf16(grads->dlogits, (int64_t)p->T * E, B.dl16, s);
    if (err == hipSuccess) err = launch_one_expert_offsets(B.roff, p->T, s);
    if (err == hipSuccess) err = launch_pack_plain(1, E, H, w_router, B.wr_packed, s);
    if (err == hipSuccess)
      err = launch_gemm_bf16(1, B.dl16, nullptr, B.roff, B.wr_packed, B.dxr, E, H, p->T <= 24,
                             s);
    if (err == hipSuccess) err = launch_pad_offsets(B.roff, 1, 64, B.rpoff, s);
    if (err == hipSuccess)
      err = launch_transpose_pad(B.dl16, nullptr, B.roff, B.rpoff, 1, E, B.tpad, false, B.dlT, s);
    if (err == hipSuccess)
      err = launch_transpose_pad(x, nullptr, B.roff, B.rpoff, 1, H, B.tpad, true, B.xTf, s);
    if (err == hipSuccess)
      err = launch_wgrad_bf16(B.dlT, B.xTf, B.rpoff, 1, E, H, B.tpad, false, grads->dw_router,
                              nullptr, s);
    dxr = B.dxr;
  }
  // dispatch backward: dx[t] = sum over kept slots of dxp rows (+ the router's path)
  if (err == hipSuccess)
    err = launch_combine(*p, B.dxp, nullptr, R.slot_to_row, dxr, grads->dx, s);
  // weight gradients over each expert's rows
  // (aT and dguT came with the SwiGLU backward)
  if (err == hipSuccess)
    err = launch_transpose_pad(x, R.row_token, R.offsets, B.poff, E, H, B.npad, false, B.xT, s);
  if (err == hipSuccess)
    err = launch_transpose_pad(B.dyp, nullptr, R.offsets, B.poff, E, H, B.npad, true, B.dypT, s);
  if (err == hipSuccess)
    err = launch_wgrad_bf16(B.aT, B.dypT, B.poff, E, I, H, B.npad, false, grads->dw_down,
                            nullptr, s);
  if (err == hipSuccess)
    err = launch_wgrad_bf16(B.xT, B.dguT, B.poff, E, H, 2 * I, B.npad, true, grads->dw_gate,
                            grads->dw_up, s);
  return status_of(err);
}

int moe_debug_status(uint32_t* status) {
  if (!status) return MOE_ERR_INVALID_ARG;
  *status = 0;
#ifdef MOE_DEBUG_CHECKS
  return status_of(debug_status_take(status));
#else
  return MOE_ERR_UNSUPPORTED;
#endif
}

size_t moe_layer_chunked_workspace_bytes(const moe_problem* p, int32_t chunk_tokens,
                                         int32_t shared_I) {
  if (chunked_check(p, chunk_tokens, shared_I) != MOE_OK) return 0;
  Carve c(nullptr);
  carve_chunked(c, *p, chunk_tokens, shared_I);
  return c.used;
}

int moe_layer_chunked(const moe_problem* p, const void* x, const float* logits,
                      const void* packed_gate_up, const void* packed_down,
                      const moe_shared_expert* shared, int32_t chunk_tokens, void* y, void* ws,
                      size_t ws_bytes, void* stream, void* aux_stream) {
  const int shared_I = shared ? shared->I : 0;
  int st = chunked_check(p, chunk_tokens, shared_I);
  if (st != MOE_OK) return st;
  if (!x || !logits || !packed_gate_up || !packed_down || !y) return MOE_ERR_INVALID_ARG;
  if (shared && (!shared->packed_gate_up || !shared->packed_down ||
                 !aligned16(shared->packed_gate_up) || !aligned16(shared->packed_down)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(packed_gate_up) || !aligned16(packed_down))
    return MOE_ERR_INVALID_ARG;
  {
    moe_problem ps = shared_problem(*p, p->T, std::max(shared_I, 1));
    if (aliased({{y, act_rows(*p, p->T, p->H)}, {ws, ws_bytes}},
                {{x, act_rows(*p, p->T, p->H)}, {logits, (size_t)p->T * p->E * 4},
                 {packed_gate_up, moe_packed_bytes(p, MOE_W_GATE_UP)},
                 {packed_down, moe_packed_bytes(p, MOE_W_DOWN)},
                 {shared ? shared->packed_gate_up : nullptr, moe_packed_bytes(&ps, MOE_W_GATE_UP)},
                 {shared ? shared->packed_down : nullptr, moe_packed_bytes(&ps, MOE_W_DOWN)}}))
      return MOE_ERR_INVALID_ARG;
  }
  const size_t need = moe_layer_chunked_workspace_bytes(p, chunk_tokens, shared_I);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255) != 0) return MOE_ERR_INVALID_ARG;
  Carve c(ws);
  ChunkScratch S = carve_chunked(c, *p, chunk_tokens, shared_I);
  if (c.used > ws_bytes) return MOE_ERR_WORKSPACE;

  hipStream_t s = as_stream(stream);
  hipStream_t aux = aux_stream ? as_stream(aux_stream) : s;
  const bool two = aux != s;
  hipEvent_t ev[5] = {};  // route done, layout set 0/1 ready, layout set 0/1 free again
  hipError_t err = hipSuccess;
  if (two)
    for (int i = 0; i < 5 && err == hipSuccess; ++i)
      err = hipEventCreateWithFlags(&ev[i], hipEventDisableTiming);
  const size_t eb = elem_bytes(p->act_dtype);
  const char* xb = static_cast<const char*>(x);
  char* yb = static_cast<char*>(y);

  // routing and the capacity over all T tokens: the result does not depend on the chunking
  if (err == hipSuccess) err = run_route(*p, logits, 1, 1, S.ids, S.w, S.keep, S.rank, s);
  if (err == hipSuccess && two) err = hipEventRecord(ev[0], s);
  if (err == hipSuccess && two) err = hipStreamWaitEvent(aux, ev[0], 0);
  const int nchunks = div_up(p->T, chunk_tokens);
  // kernel families of the whole layer, so that no row's result depends on the chunking
  const bool dec = ffn_use_decode(*p);
  const bool dec_shared = ffn_use_decode(shared_problem(*p, p->T, std::max(shared_I, 1)));
  for (int ci = 0; ci < nchunks && err == hipSuccess; ++ci) {
    const int t0 = ci * chunk_tokens;
    const int n = std::min(chunk_tokens, p->T - t0);
    const ChunkSet& L = S.set[ci & 1];
    moe_problem pc = *p;
    pc.T = n;
    // aux: the chunk's layout (and its shared-expert rows), once set ci & 1 is free again
    if (two && ci >= 2) err = hipStreamWaitEvent(aux, ev[3 + (ci & 1)], 0);
    if (err == hipSuccess)
      err = run_dispatch(pc, xb + (size_t)t0 * p->H * eb, S.ids + (size_t)t0 * p->k,
                         p->capacity > 0 ? S.keep + (size_t)t0 * p->k : nullptr, L.counts,
                         L.offsets, L.row_token, L.slot_to_row, nullptr, L.rank, aux);
    if (err == hipSuccess && shared_I > 0) {
      moe_problem ps = shared_problem(*p, n, shared_I);
      err = launch_one_expert_offsets(L.s_off, n, aux);
      if (err == hipSuccess)
        err = run_gate_up(ps, xb + (size_t)t0 * p->H * eb, nullptr, L.s_off,
                          shared->packed_gate_up, L.s_ffn.a, L.s_ffn, dec_shared, aux);
      if (err == hipSuccess)
        err = run_down(ps, L.s_ffn.a, L.s_off, shared->packed_down, L.ys, dec_shared, aux);
    }
    if (err == hipSuccess && two) err = hipEventRecord(ev[1 + (ci & 1)], aux);
    // main: the routed experts of the chunk and its combine
    if (err == hipSuccess && two) err = hipStreamWaitEvent(s, ev[1 + (ci & 1)], 0);
    if (err == hipSuccess)
      err = run_gate_up(pc, xb + (size_t)t0 * p->H * eb, L.row_token, L.offsets,
                        packed_gate_up, S.ffn.a, S.ffn, dec, s);
    if (err == hipSuccess) err = run_down(pc, S.ffn.a, L.offsets, packed_down, S.yp, dec, s);
    if (err == hipSuccess)
      err = launch_combine(pc, S.yp, S.w + (size_t)t0 * p->k, L.slot_to_row,
                           shared_I > 0 ? L.ys : nullptr, yb + (size_t)t0 * p->H * eb, s);
    if (err == hipSuccess && two) err = hipEventRecord(ev[3 + (ci & 1)], s);
  }
  // events are released once the work recorded on them has completed
  for (int i = 0; i < 5; ++i)
    if (ev[i]) (void)hipEventDestroy(ev[i]);
  return status_of(err);
}

}  // extern "C"
