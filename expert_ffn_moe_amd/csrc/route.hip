// Top-k routing (LightLLM PR #1687, call-order paragraph: top-k in the logical expert
// space, `norm_topk_prob` renormalisation, grouped top-k inside `experts()`).  One
// wavefront per token.
//
// Selection: each lane holds the logits of experts lane, lane+64, ...; k rounds of a
// wavefront max over 64-bit keys (order-preserving logit bits << 32 | ~expert) pick the
// experts in slot order, ties to the lower expert index (+0 and -0 compare equal).
//
// Weights: a specified fp32 arithmetic, reproducible bit for bit on any IEEE machine:
//   m = largest logit;  e_j = EXP(l_j - m)  (Cody-Waite reduction + degree-7 Taylor
//   polynomial, fused multiply-adds);  S = left-to-right fp32 sum of e_j over the
//   slots (or of EXP(l_e - m) over all experts e = 0..E-1 without renormalisation);
//   w_j = e_j / S with IEEE division.  No contraction anywhere in this file.
#include "moe_internal.h"
#include "wave.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

// Constants of the exponential, as fp32 bit patterns:
//   1/ln2; ln2 truncated to 15 significant bits (so n*head is exact for |n| <= 126);
//   ln2 - head; Taylor coefficients 1/i! rounded to fp32.
constexpr uint32_t kInvLn2Bits = 0x3fb8aa3bu;
constexpr uint32_t kLn2HeadBits = 0x3f317200u;
constexpr uint32_t kLn2TailBits = 0x35bfbe8eu;
constexpr uint32_t kTaylorBits[8] = {0x3f800000u, 0x3f800000u, 0x3f000000u, 0x3e2aaaabu,
                                     0x3d2aaaabu, 0x3c088889u, 0x3ab60b61u, 0x39500d01u};

__device__ __forceinline__ float bits_f(uint32_t u) { return __builtin_bit_cast(float, u); }

// exp(x) for x <= 0; x < -87 gives +0.  Never subnormal.
__device__ __forceinline__ float route_exp(float x) {
  if (x < -87.0f) return 0.0f;
  const float n = __builtin_rintf(x * bits_f(kInvLn2Bits));
  float r = __builtin_fmaf(-n, bits_f(kLn2HeadBits), x);
  r = __builtin_fmaf(-n, bits_f(kLn2TailBits), r);
  float q = bits_f(kTaylorBits[7]);
#pragma unroll
  for (int i = 6; i >= 0; --i) q = __builtin_fmaf(q, r, bits_f(kTaylorBits[i]));
  return __builtin_amdgcn_ldexpf(q, (int)n);
}

// Order-preserving map of fp32 (with -0 folded into +0) to uint32.
__device__ __forceinline__ uint32_t ordered_bits(float l) {
  uint32_t u = __float_as_uint(l == 0.0f ? 0.0f : l);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Selection and weights of one token whose logits the wavefront holds (lane: experts
// lane, lane + 64, ...; lv[i] ignored for lane + 64 i >= E).  Group limit (n_group > 1 and
// topk_group < n_group): groups of gs = E / n_group consecutive experts; topk_group rounds
// of a wavefront max over the keys of experts in groups not yet taken pick the groups in
// order of their best logit (ties: the lower expert id, hence the lower group); experts
// outside the taken groups are then removed before the k selection rounds.
template <int EPL>
__device__ __forceinline__ void select_token(const float (&lv)[EPL], int E, int k, int renorm,
                                             int n_group, int topk_group, int lane, size_t o,
                                             int32_t* __restrict__ ids, float* __restrict__ w,
                                             uint8_t* __restrict__ keep) {
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = e < E ? ((uint64_t)ordered_bits(lv[i]) << 32) | (uint32_t)(~(uint32_t)e) : 0;
  }
  if (n_group > 1 && topk_group < n_group) {  // wave-uniform
    const int gs = E / n_group;
    int grp[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) grp[i] = (lane + 64 * i) / gs;
    uint64_t taken = 0;  // bit g: group g taken (n_group <= 64)
    for (int r = 0; r < topk_group; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (!((taken >> grp[i]) & 1)) best = max_u64(best, key[i]);
      best = wave_max_u64(best);
      taken |= (uint64_t)1 << ((int)(~(uint32_t)best) / gs);
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (!((taken >> grp[i]) & 1)) key[i] = 0;
  }

  uint64_t mine = 0;  // lane j ends with the key chosen in round j
  for (int j = 0; j < k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = max_u64(best, key[i]);
    best = wave_max_u64(best);
    if (lane == j) mine = best;
    const uint32_t ew = ~(uint32_t)best;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if ((uint32_t)(lane + 64 * i) == ew) key[i] = 0;
  }

  const float l = unordered_bits((uint32_t)(mine >> 32));
  const int e = (int)(~(uint32_t)mine);
  const float m = __shfl(l, 0, 64);
  const float ex = (lane < k) ? route_exp(l - m) : 0.0f;
  float s = 0.0f;
  if (renorm) {
    for (int j = 0; j < k; ++j) s = s + __shfl(ex, j, 64);
  } else {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const float ev = (lane + 64 * i < E) ? route_exp(lv[i] - m) : 0.0f;
      const int n = min(64, E - 64 * i);
      for (int src = 0; src < n; ++src)
        s = s + __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(ev), src));
    }
  }
  if (lane < k) {
    ids[o + lane] = e;
    w[o + lane] = ex / s;
    keep[o + lane] = 1;
  }
}

// One wavefront per token.  The logits are the sum, in plane order, of S fp32 planes
// (S = 1: the logits themselves; S > 1: the router GEMM's split-K partial sums), written
// to logits_out if it is not NULL, then selected.
template <int EPL>  // experts per lane: E <= 64 * EPL
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int S,
                                                    size_t plane, int T, int E, int k,
                                                    int renorm, int n_group, int topk_group,
                                                    float* __restrict__ logits_out,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w,
                                                    uint8_t* __restrict__ keep) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform
  const float* row = logits + (size_t)t * E;
  float lv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    float v = 0.0f;
    if (e < E) {
      v = row[e];
#pragma unroll 8
      for (int q = 1; q < S; ++q) v = v + row[q * plane + e];
      if (logits_out) logits_out[(size_t)t * E + e] = v;
    }
    lv[i] = v;
  }
  select_token<EPL>(lv, E, k, renorm, n_group, topk_group, lane, (size_t)t * k, ids, w, keep);
}

// Gradient of the logits from the gradient of the routing weights (dw = 0 for dropped
// slots); the selection itself carries none.  One wavefront per token.
//   renormalised: dl_j = w_j (dw_j - sum_i w_i dw_i) on the k selected experts, 0 elsewhere
//   plain softmax: dl_e = p_e ([e selected] dw_e - sum_i w_i dw_i), p the softmax over all E
// (p recomputed with the routing's exponential; sums in slot / expert order, fp32).
template <int EPL>
__global__ __launch_bounds__(256) void route_bwd_kernel(const float* __restrict__ logits,
                                                        const int32_t* __restrict__ ids,
                                                        const float* __restrict__ w,
                                                        const float* __restrict__ dw, int T,
                                                        int E, int k, int renorm,
                                                        float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform
  const size_t o = (size_t)t * k;
  float inner = 0.0f;
  for (int j = 0; j < k; ++j) inner = inner + w[o + j] * dw[o + j];
  float p[EPL], d[EPL];
  if (renorm) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) p[i] = 0.0f, d[i] = 0.0f;
  } else {
    const float* row = logits + (size_t)t * E;
    float lv[EPL];
    float m = -3.402823466e38f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      lv[i] = e < E ? row[e] : -3.402823466e38f;
      m = fmaxf(m, lv[i]);
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) m = fmaxf(m, __shfl_xor(m, sh, 64));
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      p[i] = (lane + 64 * i < E) ? route_exp(lv[i] - m) : 0.0f;
      const int n = min(64, E - 64 * i);
      for (int src = 0; src < n; ++src)
        s = s + __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(p[i]), src));
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      p[i] = p[i] / s;
      d[i] = -p[i] * inner;
    }
  }
  for (int j = 0; j < k; ++j) {
    const int e = ids[o + j];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i == e)
        d[i] = renorm ? w[o + j] * (dw[o + j] - inner) : d[i] + p[i] * dw[o + j];
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + 64 * i < E) dl[(size_t)t * E + lane + 64 * i] = d[i];
}

template <int EPL>
hipError_t launch_route_bwd_t(const moe_problem& p, const float* logits, const int32_t* ids,
                              const float* w, const float* dw, float* dl, hipStream_t s) {
  hipLaunchKernelGGL(route_bwd_kernel<EPL>, dim3(div_up(p.T, 4)), dim3(256), 0, s, logits, ids,
                     w, dw, p.T, p.E, p.k, p.renormalize, dl);
  return hipGetLastError();
}

template <int EPL>
hipError_t launch_route_t(const moe_problem& p, const float* logits, int S, int n_group,
                          int topk_group, float* logits_out, int32_t* ids, float* w,
                          uint8_t* keep, hipStream_t s) {
  dim3 grid(div_up(p.T, 4));
  hipLaunchKernelGGL(route_kernel<EPL>, grid, dim3(256), 0, s, logits, S,
                     (size_t)p.T * p.E, p.T, p.E, p.k, p.renormalize, n_group, topk_group,
                     logits_out, ids, w, keep);
  return hipGetLastError();
}

hipError_t launch_select(const moe_problem& p, const float* logits, int S, int n_group,
                         int topk_group, float* logits_out, int32_t* ids, float* w,
                         uint8_t* keep, hipStream_t s) {
  if (p.E <= 64)
    return launch_route_t<1>(p, logits, S, n_group, topk_group, logits_out, ids, w, keep, s);
  if (p.E <= 128)
    return launch_route_t<2>(p, logits, S, n_group, topk_group, logits_out, ids, w, keep, s);
  if (p.E <= 256)
    return launch_route_t<4>(p, logits, S, n_group, topk_group, logits_out, ids, w, keep, s);
  if (p.E <= 512)
    return launch_route_t<8>(p, logits, S, n_group, topk_group, logits_out, ids, w, keep, s);
  return launch_route_t<16>(p, logits, S, n_group, topk_group, logits_out, ids, w, keep, s);
}

// ---------------------------------------------------------------------------------------
// Router front-end: logits = x W_r^T (bf16 operands, fp32 accumulation on the matrix
// cores), split along H into S slices so that the grid fills the chip whatever T is; the
// selection kernel above sums the S partial planes in order before selecting (so the
// split-K reduction and the selection are one launch).
//
// A block takes R = 16 W rows (W wavefronts) and all E <= 256 experts for one slice of H:
// wavefront w computes its 16 rows against every expert with v_mfma_f32_16x16x32_bf16
// (E / 16 accumulators of 4 registers).  Its x rows stream straight from memory, one chunk
// of 64 ahead (no other wavefront needs them); the gate weights, shared by all wavefronts,
// go through LDS in chunks of 64 along H (E rows x 128 bytes, 16-byte pieces swizzled by
// (e >> 1) & 7 so that the 16 rows of one read touch every bank once), double-buffered
// with the next chunk held in registers.
// ---------------------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_r __attribute__((ext_vector_type(4)));

constexpr int kRouterMaxE = 256;

__device__ __forceinline__ int wr_slot(int e, int piece) { return e * 8 + (piece ^ ((e >> 1) & 7)); }

template <int NT, int W>  // E = 16 NT experts, W wavefronts (16 W rows)
__global__ __launch_bounds__(64 * W) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ wr,
                                                             int T, int H, int cps,
                                                             float* __restrict__ part) {
  constexpr int E = 16 * NT;
  constexpr int kPieces = E * 8;                        // 16-byte pieces per chunk
  constexpr int kPer = (kPieces + 64 * W - 1) / (64 * W);  // per thread
  __shared__ u32x4_r lds[2 * E * 8];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int row0 = blockIdx.x * 16 * W;
  const int c0 = blockIdx.y * cps;  // first chunk of this slice
  const int ar = min(row0 + 16 * wave + (lane & 15), T - 1);
  const uint16_t* ap = x + (size_t)ar * H + 64 * c0 + 8 * (lane >> 4);
  const uint16_t* wp = wr + 64 * c0;

  f32x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{};
  // (vector types throughout: with the struct uint4, pre[] was kept in scratch memory)
  u32x4_r pre[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = tid + 64 * W * j;
    if (q < kPieces) pre[j] = *(const u32x4_r*)(wp + (size_t)(q >> 3) * H + 8 * (q & 7));
  }
  // x chunks c, c + 1, c + 2 in registers (HBM latency spans a few chunks of MFMAs)
  u32x4_r xa[3][2];
#pragma unroll
  for (int d = 0; d < 3; ++d) {
    const int cd = min(d, cps - 1);
    xa[d][0] = *(const u32x4_r*)(ap + 64 * cd);
    xa[d][1] = *(const u32x4_r*)(ap + 64 * cd + 32);
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int q = tid + 64 * W * j;
    if (q < kPieces) lds[wr_slot(q >> 3, q & 7)] = pre[j];
  }
  __syncthreads();
  for (int c = 0; c < cps; ++c) {
    const int buf = c & 1;
    const int cn = min(c + 1, cps - 1);  // the last iteration reloads its own chunk
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int q = tid + 64 * W * j;
      if (q < kPieces)
        pre[j] = *(const u32x4_r*)(wp + (size_t)(q >> 3) * H + 64 * cn + 8 * (q & 7));
    }
    const int c3 = min(c + 3, cps - 1);
    const u32x4_r n0 = *(const u32x4_r*)(ap + 64 * c3);
    const u32x4_r n1 = *(const u32x4_r*)(ap + 64 * c3 + 32);
    const u32x4_r* b = lds + buf * (E * 8);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, xa[0][ks]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4_r bv = b[wr_slot(16 * t + (lane & 15), 4 * ks + (lane >> 4))];
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, bv),
                                                          acc[t], 0, 0, 0);
      }
    }
    u32x4_r* nb = lds + (buf ^ 1) * (E * 8);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int q = tid + 64 * W * j;
      if (q < kPieces) nb[wr_slot(q >> 3, q & 7)] = pre[j];
    }
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      xa[d][0] = xa[d + 1][0];
      xa[d][1] = xa[d + 1][1];
    }
    xa[2][0] = n0;
    xa[2][1] = n1;
    __syncthreads();
  }
  // partial logits of this slice: accumulator element i of lane l is row
  // 4 (l / 16) + i of the wavefront's 16, expert 16 t + l % 16
  float* out = part + (size_t)blockIdx.y * T * E;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row0 + 16 * wave + 4 * (lane >> 4) + i;
    if (r < T) {
#pragma unroll
      for (int t = 0; t < NT; ++t) out[(size_t)r * E + 16 * t + (lane & 15)] = acc[t][i];
    }
  }
}

template <int NT>
hipError_t launch_router_gemm_t(const moe_problem& p, const RouterPlan& plan, const void* x,
                                const void* wr, float* part, hipStream_t s) {
  const dim3 grid(div_up(p.T, plan.rows), plan.split);
  const int cps = p.H / 64 / plan.split;
  if (plan.rows == 128)
    hipLaunchKernelGGL((router_gemm_kernel<NT, 8>), grid, dim3(512), 0, s,
                       (const uint16_t*)x, (const uint16_t*)wr, p.T, p.H, cps, part);
  else
    hipLaunchKernelGGL((router_gemm_kernel<NT, 4>), grid, dim3(256), 0, s,
                       (const uint16_t*)x, (const uint16_t*)wr, p.T, p.H, cps, part);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const moe_problem& p, const float* logits, int n_group, int topk_group,
                        int32_t* ids, float* w, uint8_t* keep, hipStream_t s) {
  return launch_select(p, logits, 1, n_group, topk_group, nullptr, ids, w, keep, s);
}

hipError_t launch_route_bwd(const moe_problem& p, const float* logits, const int32_t* ids,
                            const float* w, const float* dw, float* dl, hipStream_t s) {
  if (p.E <= 64) return launch_route_bwd_t<1>(p, logits, ids, w, dw, dl, s);
  if (p.E <= 128) return launch_route_bwd_t<2>(p, logits, ids, w, dw, dl, s);
  if (p.E <= 256) return launch_route_bwd_t<4>(p, logits, ids, w, dw, dl, s);
  if (p.E <= 512) return launch_route_bwd_t<8>(p, logits, ids, w, dw, dl, s);
  return launch_route_bwd_t<16>(p, logits, ids, w, dw, dl, s);
}

bool router_supported(const moe_problem& p) {
  return p.act_dtype == MOE_BF16 && p.E % 16 == 0 && p.E <= kRouterMaxE && p.H % 64 == 0;
}

// Rows per block, then the smallest split of the H / 64 chunks (a divisor, so slices are
// equal) that gives at least 256 blocks; at most 16 slices (the selection kernel reads
// every partial plane).
RouterPlan router_plan(const moe_problem& p) {
  RouterPlan plan;
  // 128 rows (8 wavefronts) from 2048 tokens up: 256-row blocks of 16 wavefronts, which
  // share each gate chunk among twice the rows, measured 10% slower on the DSV3 shape
  // (T = 16384: 83 vs 75 us)
  plan.rows = p.T >= 2048 ? 128 : 64;
  const int tiles = div_up(p.T, plan.rows);
  const int nch = p.H / 64;
  plan.split = 1;
  for (int d = 1; d <= nch && d <= 16; ++d) {
    if (nch % d) continue;
    plan.split = d;
    if ((int64_t)tiles * d >= 256) break;
  }
  return plan;
}

hipError_t launch_router(const moe_problem& p, const void* x, const void* wr, int n_group,
                         int topk_group, float* part, float* logits, int32_t* ids, float* w,
                         uint8_t* keep, hipStream_t s) {
  const RouterPlan plan = router_plan(p);
  hipError_t err;
  switch (p.E / 16) {
#define MOE_ROUTER_CASE(n) \
  case n:                  \
    err = launch_router_gemm_t<n>(p, plan, x, wr, part, s); \
    break;
    MOE_ROUTER_CASE(1) MOE_ROUTER_CASE(2) MOE_ROUTER_CASE(3) MOE_ROUTER_CASE(4)
    MOE_ROUTER_CASE(5) MOE_ROUTER_CASE(6) MOE_ROUTER_CASE(7) MOE_ROUTER_CASE(8)
    MOE_ROUTER_CASE(9) MOE_ROUTER_CASE(10) MOE_ROUTER_CASE(11) MOE_ROUTER_CASE(12)
    MOE_ROUTER_CASE(13) MOE_ROUTER_CASE(14) MOE_ROUTER_CASE(15) MOE_ROUTER_CASE(16)
#undef MOE_ROUTER_CASE
    default:
      return hipErrorInvalidValue;
  }
  if (err != hipSuccess) return err;
  return launch_select(p, part, plan.split, n_group, topk_group, logits, ids, w, keep, s);
}

}  // namespace moe
