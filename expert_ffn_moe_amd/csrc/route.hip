// Top-k routing (LightLLM PR #1687, call-order paragraph: top-k in the logical expert
// space, `norm_topk_prob` renormalisation).  One wavefront per token.
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

template <int EPL>  // experts per lane: E <= 64 * EPL
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int k, int renorm,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ w,
                                                    uint8_t* __restrict__ keep) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // wave-uniform
  const float* row = logits + (size_t)t * E;

  uint64_t key[EPL];
  float lv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      lv[i] = row[e];
      key[i] = ((uint64_t)ordered_bits(lv[i]) << 32) | (uint32_t)(~(uint32_t)e);
    } else {
      lv[i] = 0.0f;
      key[i] = 0;  // below every real key
    }
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
    const size_t o = (size_t)t * k + lane;
    ids[o] = e;
    w[o] = ex / s;
    keep[o] = 1;
  }
}

template <int EPL>
hipError_t launch_route_t(const moe_problem& p, const float* logits, int32_t* ids, float* w,
                          uint8_t* keep, hipStream_t s) {
  dim3 grid(div_up(p.T, 4));
  hipLaunchKernelGGL(route_kernel<EPL>, grid, dim3(256), 0, s, logits, p.T, p.E, p.k,
                     p.renormalize, ids, w, keep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const moe_problem& p, const float* logits, int32_t* ids, float* w,
                        uint8_t* keep, hipStream_t s) {
  if (p.E <= 64) return launch_route_t<1>(p, logits, ids, w, keep, s);
  if (p.E <= 128) return launch_route_t<2>(p, logits, ids, w, keep, s);
  if (p.E <= 256) return launch_route_t<4>(p, logits, ids, w, keep, s);
  if (p.E <= 512) return launch_route_t<8>(p, logits, ids, w, keep, s);
  return launch_route_t<16>(p, logits, ids, w, keep, s);
}

}  // namespace moe
