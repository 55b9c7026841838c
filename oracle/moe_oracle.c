/*
 * moe_oracle.c -- plain, slow, obviously-correct CPU oracle for one GPU's share
 * of an expert-parallel MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) may link, load or call this file.  It shares no code,
 * header, constant table or helper with the HIP kernels.
 *
 * The pages define the method in prose only; each function below names the
 * passage it follows:
 *   [P1] docs.axolotl.ai, "integrations.expert_parallel.args", attribute
 *        table, row `expert_parallel_token_capacity` (per-expert cap; the
 *        lowest-weight excess (token, expert) assignments are dropped; None
 *        means no cap).
 *   [P4] LightLLM PR #1687 page, PR body ("调用顺序" / call-order paragraph):
 *        top-k only in the logical expert space, optional renormalisation
 *        (`norm_topk_prob`), expert prefix-sum ("psum") layout consumed by the
 *        grouped GEMM, SwiGLU (`silu_and_mul_...`) after the gate/up GEMM,
 *        and a decode step that reduces expert outputs back to dense output.
 *   [P5] research-vault claim card, "Evidence": in pure DP+EP the one
 *        communication pattern is the all-to-all that routes tokens to
 *        experts; on one GPU that exchange is the local permutation below.
 *
 * Arithmetic conventions (readings recorded with the oracle):
 *   - Routing weights are fp32 and computed in a fixed, specified way so that
 *     a second implementation can reproduce them bit for bit: a Cody-Waite
 *     reduced, Taylor-polynomial exp (orc_exp), a left-to-right fp32 sum and
 *     IEEE division.  Build with -ffp-contract=off and without fast-math.
 *   - The FFN and the combine accumulate in fp64 (the oracle's precision).
 *
 * Parity pins for every function live in tests/ (brute force, closed forms,
 * invariants, special cases).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_BF16 1

/* ------------------------------------------------------------------------ */
/* Specified fp32 exponential.                                              */
/*                                                                          */
/* Range reduction after Cody & Waite (Software Manual for the Elementary   */
/* Functions, 1980): x = n*ln2 + r with n = nearest integer to x/ln2 and    */
/* ln2 split into a head with trailing zero bits plus a tail.  exp(r) is    */
/* the degree-7 Taylor polynomial in Horner form with fused multiply-adds,  */
/* coefficients 1/i! rounded to fp32.  Defined for x <= 0 (the only inputs  */
/* routing produces); x < -87 returns +0.  Results are never subnormal.     */
/* ------------------------------------------------------------------------ */
static const float ORC_INV_LN2 = 0x1.715476p+0f;   /* fp32(1/ln 2)            */
static const float ORC_LN2_HEAD = 0x1.62e4p-1f;    /* ln 2 cut to 15 bits     */
static const float ORC_LN2_TAIL = 0x1.7f7d1cp-20f; /* fp32(ln 2 - head)       */

static float orc_taylor_coef(int i) {
  double f = 1.0;
  for (int j = 2; j <= i; ++j) f *= (double)j;
  return (float)(1.0 / f);
}

float orc_exp(float x) {
  if (x < -87.0f) return 0.0f;
  float n = nearbyintf(x * ORC_INV_LN2);
  float r = fmaf(-n, ORC_LN2_HEAD, x);
  r = fmaf(-n, ORC_LN2_TAIL, r);
  float p = orc_taylor_coef(7);
  for (int i = 6; i >= 0; --i) p = fmaf(p, r, orc_taylor_coef(i));
  return ldexpf(p, (int)n);
}

/* Maximum error of orc_exp, in units of the last place of the exact result,
 * over every fp32 x in [lo, hi] (lo <= hi <= 0), against libm's fp64 exp. */
double orc_exp_max_ulp(float lo, float hi, float* worst_x) {
  uint32_t blo, bhi;
  memcpy(&blo, &hi, 4); /* negative floats: larger magnitude = larger bits */
  memcpy(&bhi, &lo, 4);
  if (hi == 0.0f) blo = 0x80000000u;
  double worst = 0.0;
  float wx = 0.0f;
#pragma omp parallel
  {
    double lw = 0.0;
    float lx = 0.0f;
#pragma omp for schedule(static)
    for (int64_t b = (int64_t)blo; b <= (int64_t)bhi; ++b) {
      uint32_t u = (uint32_t)b;
      float x;
      memcpy(&x, &u, 4);
      double ref = exp((double)x);
      double got = (double)orc_exp(x);
      int ex;
      frexp(ref, &ex); /* ref in [2^(ex-1), 2^ex) */
      double ulp = ldexp(1.0, ex - 24);
      double err = fabs(got - ref) / ulp;
      if (err > lw) { lw = err; lx = x; }
    }
#pragma omp critical
    {
      if (lw > worst) { worst = lw; wx = lx; }
    }
  }
  if (worst_x) *worst_x = wx;
  return worst;
}

/* ------------------------------------------------------------------------ */
/* Routing: top-k over the router logits of each token, softmax weights    */
/* restricted to the chosen experts.  [P4] call-order paragraph: selection  */
/* happens in the logical expert space; `norm_topk_prob` renormalises the   */
/* top-k weights to sum to 1.                                               */
/*                                                                          */
/* Selection order: logit descending, ties to the lower expert index.  The  */
/* softmax is strictly increasing in the logit, so the k largest softmax    */
/* probabilities are the k largest logits.                                  */
/* Weights with renormalisation: with m the largest logit,                  */
/*   w_j = exp(l_j - m) / (((e_0 + e_1) + e_2) + ... + e_{k-1})             */
/* (the full softmax denominator cancels).  Without renormalisation the     */
/* divisor is the left-to-right fp32 sum of exp(l_e - m) over e = 0..E-1.   */
/* ------------------------------------------------------------------------ */
void orc_route(int T, int E, int k, int renormalize, const float* logits,
               int32_t* topk_ids, float* topk_w) {
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
    int32_t* ids = topk_ids + (size_t)t * k;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: ties keep lower e */
      }
      taken[best] = 1;
      ids[j] = best;
    }
    free(taken);
    float m = l[ids[0]];
    float ex[64];
    float s = 0.0f;
    for (int j = 0; j < k; ++j) {
      ex[j] = orc_exp(l[ids[j]] - m);
      s = s + ex[j];
    }
    if (!renormalize) {
      s = 0.0f;
      for (int e = 0; e < E; ++e) s = s + orc_exp(l[e] - m);
    }
    for (int j = 0; j < k; ++j) topk_w[(size_t)t * k + j] = ex[j] / s;
  }
}

/* ------------------------------------------------------------------------ */
/* Group-limited selection.  [P4] call-order paragraph: `experts()` keeps   */
/* doing grouped top-k inside the layer for some models; the pages do not   */
/* give the group rule.  Reading (the plainest one):                        */
/*   - the E experts form n_group equal groups of consecutive ids;          */
/*   - a group's score is the largest logit in it;                          */
/*   - the topk_group groups with the largest scores are taken, ties to     */
/*     the lower group index;                                               */
/*   - the k largest logits among the experts of the taken groups are       */
/*     selected (slot order: logit descending, ties to the lower id).       */
/* Weights exactly as in orc_route: with renormalisation over the k chosen  */
/* (m, the largest chosen logit, is the largest logit overall: its group    */
/* always has the top score); without, the plain softmax over all E.        */
/* n_group = 1 is orc_route.                                                */
/* ------------------------------------------------------------------------ */
void orc_route_grouped(int T, int E, int k, int renormalize, int n_group, int topk_group,
                       const float* logits, int32_t* topk_ids, float* topk_w) {
  const int gs = E / n_group;
  unsigned char* allowed = (unsigned char*)malloc((size_t)E);
  unsigned char* gtaken = (unsigned char*)malloc((size_t)n_group);
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  for (int t = 0; t < T; ++t) {
    const float* l = logits + (size_t)t * E;
    /* group scores, then the topk_group best groups */
    memset(gtaken, 0, (size_t)n_group);
    memset(allowed, 0, (size_t)E);
    for (int r = 0; r < topk_group; ++r) {
      int bg = -1;
      float bs = 0.0f;
      for (int g = 0; g < n_group; ++g) {
        if (gtaken[g]) continue;
        float sc = l[g * gs];
        for (int e = g * gs + 1; e < (g + 1) * gs; ++e)
          if (l[e] > sc) sc = l[e];
        if (bg < 0 || sc > bs) { bg = g; bs = sc; } /* strict: ties keep the lower g */
      }
      gtaken[bg] = 1;
      for (int e = bg * gs; e < (bg + 1) * gs; ++e) allowed[e] = 1;
    }
    /* top-k among the allowed experts */
    memset(taken, 0, (size_t)E);
    int32_t* ids = topk_ids + (size_t)t * k;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (!allowed[e] || taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      ids[j] = best;
    }
    /* weights */
    float m = l[ids[0]];
    float ex[64];
    float s = 0.0f;
    for (int j = 0; j < k; ++j) {
      ex[j] = orc_exp(l[ids[j]] - m);
      s = s + ex[j];
    }
    if (!renormalize) {
      s = 0.0f;
      for (int e = 0; e < E; ++e) s = s + orc_exp(l[e] - m);
    }
    for (int j = 0; j < k; ++j) topk_w[(size_t)t * k + j] = ex[j] / s;
  }
  free(allowed);
  free(gtaken);
  free(taken);
}

/* ------------------------------------------------------------------------ */
/* Router logits.  [P4] call-order paragraph: the layer's own `experts()`   */
/* path computes the routing from the hidden states (the gate); the plain   */
/* reading is a linear gate without bias: logits[t, e] = sum_h x[t, h] *    */
/* W_r[e, h], W_r stored [E, H] (one row of H weights per expert).  fp64    */
/* accumulation, h ascending.                                               */
/* ------------------------------------------------------------------------ */
static inline double orc_load(const void* p, size_t i, int dtype);

void orc_router_logits(int T, int H, int E, int dtype, const void* x, const void* w_router,
                       double* logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += orc_load(x, (size_t)t * H + h, dtype) * orc_load(w_router, (size_t)e * H + h, dtype);
      logits[(size_t)t * E + e] = acc;
    }
}

/* ------------------------------------------------------------------------ */
/* Per-expert capacity.  [P1] `expert_token_capacity` row: at most C        */
/* (token, expert) assignments per expert per forward; the lowest-weight    */
/* excess ones are dropped.  Order: weight descending, ties to the lower    */
/* token index.  Weights are the routing weights carried into the combine.  */
/* keep[t*k+j] = 1 for kept, 0 for dropped.  C <= 0 means no cap.           */
/* ------------------------------------------------------------------------ */
typedef struct {
  float w;
  int32_t t;
  int32_t slot;
} orc_cand;

static int orc_cand_cmp(const void* pa, const void* pb) {
  const orc_cand* a = (const orc_cand*)pa;
  const orc_cand* b = (const orc_cand*)pb;
  if (a->w > b->w) return -1;
  if (a->w < b->w) return 1;
  return (a->t < b->t) ? -1 : (a->t > b->t);
}

void orc_capacity(int T, int E, int k, int C, const int32_t* topk_ids,
                  const float* topk_w, uint8_t* keep) {
  for (size_t s = 0; s < (size_t)T * k; ++s) keep[s] = 1;
  if (C <= 0) return;
  orc_cand* c = (orc_cand*)malloc(sizeof(orc_cand) * (size_t)T * k + 1);
  for (int e = 0; e < E; ++e) {
    size_t n = 0;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (topk_ids[(size_t)t * k + j] == e) {
          c[n].w = topk_w[(size_t)t * k + j];
          c[n].t = t;
          c[n].slot = t * k + j;
          ++n;
        }
    if (n <= (size_t)C) continue;
    qsort(c, n, sizeof(orc_cand), orc_cand_cmp);
    for (size_t i = (size_t)C; i < n; ++i) keep[c[i].slot] = 0;
  }
  free(c);
}

/* ------------------------------------------------------------------------ */
/* Expert-contiguous layout.  [P4] "Decode already runs on the expert       */
/* prefix-sum layout" and `use_psum_layout=True`: rows grouped by expert,   */
/* addressed by the prefix sums of the per-expert counts.  [P5]: on one GPU */
/* this permutation stands in for the dispatch all-to-all.                  */
/*   counts[e]  = kept assignments to e                                     */
/*   offsets    = exclusive scan of counts, offsets[E] = N                  */
/*   rows inside a segment in ascending token order (stable counting sort   */
/*   of the row-major (t, j) list by expert id)                             */
/*   row_token[r] = token of row r; slot_to_row[t*k+j] = row, -1 if dropped */
/* Returns N.                                                               */
/* ------------------------------------------------------------------------ */
int orc_layout(int T, int E, int k, const int32_t* topk_ids, const uint8_t* keep,
               int32_t* counts, int32_t* offsets, int32_t* row_token,
               int32_t* slot_to_row) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (size_t s = 0; s < (size_t)T * k; ++s)
    if (!keep || keep[s]) counts[topk_ids[s]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      size_t s = (size_t)t * k + j;
      if (keep && !keep[s]) {
        slot_to_row[s] = -1;
        continue;
      }
      int e = topk_ids[s];
      int r = offsets[e] + fill[e];
      fill[e] += 1;
      row_token[r] = t;
      slot_to_row[s] = r;
    }
  free(fill);
  return offsets[E];
}

/* Row gather (local dispatch): xp[r, :] = x[row_token[r], :], byte copy. */
void orc_gather(int N, int H, int elem_bytes, const void* x, const int32_t* row_token,
                void* xp) {
  size_t rb = (size_t)H * elem_bytes;
  for (int r = 0; r < N; ++r)
    memcpy((char*)xp + (size_t)r * rb, (const char*)x + (size_t)row_token[r] * rb, rb);
}

/* ------------------------------------------------------------------------ */
/* Expert FFN.  [P4] grouped GEMM on the psum layout, then                  */
/* `silu_and_mul`: for a row x of expert e,                                 */
/*   g = x . Wg[e],  u = x . Wu[e]      (Wg, Wu: [H, I] row-major)          */
/*   a = silu(g) * u,  silu(z) = z / (1 + exp(-z))                          */
/*   y = a . Wd[e]                      (Wd: [I, H] row-major)              */
/* Inputs are upcast exactly; every sum runs in fp64 in index order.        */
/*                                                                          */
/* rows: nrows rows, row i belongs to expert row_expert[i] (an index into   */
/* the weight arrays given, which may hold a subset of the experts) and has */
/* its input in xrows[i, :] (act dtype).  Outputs: yp[i, :] (fp64) and,     */
/* if a_out != NULL, a_out[i, :] (fp64).                                    */
/* ------------------------------------------------------------------------ */
static inline double orc_load(const void* p, size_t i, int dtype) {
  if (dtype == ORC_F32) return (double)((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

#define ORC_RB 32 /* rows per block sharing one pass over an expert's weights */

void orc_ffn_rows(int H, int I, int x_dtype, int w_dtype, int nrows, const int32_t* row_expert,
                  const void* xrows, const void* w_gate, const void* w_up, const void* w_down,
                  double* yp, double* a_out, int nthreads) {
  /* group rows by expert (stable), then blocks of up to ORC_RB rows */
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nrows + 1));
  int maxe = 0;
  for (int i = 0; i < nrows; ++i)
    if (row_expert[i] > maxe) maxe = row_expert[i];
  int32_t* cnt = (int32_t*)calloc((size_t)maxe + 2, sizeof(int32_t));
  for (int i = 0; i < nrows; ++i) cnt[row_expert[i] + 1] += 1;
  for (int e = 0; e <= maxe; ++e) cnt[e + 1] += cnt[e];
  int32_t* pos = (int32_t*)malloc(sizeof(int32_t) * ((size_t)maxe + 1));
  for (int e = 0; e <= maxe; ++e) pos[e] = cnt[e];
  for (int i = 0; i < nrows; ++i) order[pos[row_expert[i]]++] = i;
  /* task list: (start, len) blocks that never straddle two experts */
  int ntask = 0;
  int32_t* tstart = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nrows + maxe + 2));
  int32_t* tlen = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nrows + maxe + 2));
  for (int e = 0; e <= maxe; ++e)
    for (int s = cnt[e]; s < cnt[e + 1]; s += ORC_RB) {
      tstart[ntask] = s;
      tlen[ntask] = (cnt[e + 1] - s < ORC_RB) ? cnt[e + 1] - s : ORC_RB;
      ++ntask;
    }
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
  {
    double* g = (double*)malloc(sizeof(double) * ORC_RB * (size_t)I);
    double* u = (double*)malloc(sizeof(double) * ORC_RB * (size_t)I);
    double* wrow = (double*)malloc(sizeof(double) * (size_t)(H > I ? H : I));
    double* wrow2 = (double*)malloc(sizeof(double) * (size_t)I);
    double* y = (double*)malloc(sizeof(double) * ORC_RB * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int ti = 0; ti < ntask; ++ti) {
      int nb = tlen[ti];
      const int32_t* rows = order + tstart[ti];
      size_t e = (size_t)row_expert[rows[0]];
      memset(g, 0, sizeof(double) * ORC_RB * (size_t)I);
      memset(u, 0, sizeof(double) * ORC_RB * (size_t)I);
      memset(y, 0, sizeof(double) * ORC_RB * (size_t)H);
      for (int h = 0; h < H; ++h) {
        size_t wb = (e * (size_t)H + (size_t)h) * (size_t)I;
        for (int i = 0; i < I; ++i) {
          wrow[i] = orc_load(w_gate, wb + i, w_dtype);
          wrow2[i] = orc_load(w_up, wb + i, w_dtype);
        }
        for (int r = 0; r < nb; ++r) {
          double xv = orc_load(xrows, (size_t)rows[r] * H + h, x_dtype);
          double* gr = g + (size_t)r * I;
          double* ur = u + (size_t)r * I;
          for (int i = 0; i < I; ++i) {
            gr[i] += xv * wrow[i];
            ur[i] += xv * wrow2[i];
          }
        }
      }
      for (int r = 0; r < nb; ++r)
        for (int i = 0; i < I; ++i) {
          double z = g[(size_t)r * I + i];
          double a = z / (1.0 + exp(-z)) * u[(size_t)r * I + i];
          g[(size_t)r * I + i] = a;
          if (a_out) a_out[(size_t)rows[r] * I + i] = a;
        }
      for (int i = 0; i < I; ++i) {
        size_t wb = (e * (size_t)I + (size_t)i) * (size_t)H;
        for (int h = 0; h < H; ++h) wrow[h] = orc_load(w_down, wb + h, w_dtype);
        for (int r = 0; r < nb; ++r) {
          double av = g[(size_t)r * I + i];
          double* yr = y + (size_t)r * H;
          for (int h = 0; h < H; ++h) yr[h] += av * wrow[h];
        }
      }
      for (int r = 0; r < nb; ++r)
        memcpy(yp + (size_t)rows[r] * H, y + (size_t)r * H, sizeof(double) * (size_t)H);
    }
    free(g);
    free(u);
    free(wrow);
    free(wrow2);
    free(y);
  }
  free(order);
  free(cnt);
  free(pos);
  free(tstart);
  free(tlen);
}

/* ------------------------------------------------------------------------ */
/* Combine.  [P4] decode "reduces expert outputs into dense output": each   */
/* token's output is the weight-scaled sum of its kept expert rows, in slot */
/* order, in fp64.  A token with every slot dropped gets 0.                 */
/*   y[t, :] = sum_{j: keep} w[t, j] * yp[slot_to_row[t, j], :]             */
/* tokens: the ntok token indices to produce (y has ntok rows).             */
/* ------------------------------------------------------------------------ */
void orc_combine(int ntok, const int32_t* tokens, int H, int k, const float* topk_w,
                 const int32_t* slot_to_row, const double* yp, double* y) {
  for (int i = 0; i < ntok; ++i) {
    int t = tokens[i];
    double* yt = y + (size_t)i * H;
    for (int h = 0; h < H; ++h) yt[h] = 0.0;
    for (int j = 0; j < k; ++j) {
      int r = slot_to_row[(size_t)t * k + j];
      if (r < 0) continue;
      double w = (double)topk_w[(size_t)t * k + j];
      const double* yr = yp + (size_t)r * H;
      for (int h = 0; h < H; ++h) yt[h] += w * yr[h];
    }
  }
}

/* Element-wise orc_exp over an array (for the pins in tests/). */
void orc_exp_vec(int64_t n, const float* x, float* y) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_exp(x[i]);
}

/* ======================================================================== */
/* FP8 expert FFN ([P4] PR body: the grouped GEMMs run in FP8 with UE8M0     */
/* power-of-two scales, `silu_and_mul_psum_post_quant_fwd` quantises the    */
/* SwiGLU output on the prefix-sum layout; the PR's quantisation test       */
/* expects a scale of exactly 2^-8).  Readings recorded with the oracle:    */
/*   - element format: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7,   */
/*     3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN, largest */
/*     finite 448); conversion rounds to nearest, ties to even;             */
/*   - a scale covers a block of 32 consecutive elements along the GEMM's   */
/*     reduction dimension and is a power of two 2^e stored as the unsigned */
/*     E8M0 byte e + 127, e the smallest integer with amax <= 448 * 2^e     */
/*     (nothing saturates); an all-zero block takes e = 0;                  */
/*   - x is quantised per token row, the weights per column along the       */
/*     reduction dimension, the SwiGLU output `a` per row before the down    */
/*     projection; products accumulate in fp64 here.                        */
/* ======================================================================== */
#define ORC_QB 32

/* Value of an E4M3 code (NaN for the two NaN codes). */
double orc_e4m3_value(int code) {
  int s = (code >> 7) & 1, E = (code >> 3) & 15, M = code & 7;
  if (E == 15 && M == 7) return NAN;
  double mag = (E == 0) ? ldexp((double)M, -9) : ldexp(8.0 + M, E - 10);
  return s ? -mag : mag;
}

/* Nearest E4M3 code to v (|v| <= 448), ties to the even code; the sign is kept
 * for values that round to zero.  Plain search over the 127 non-negative
 * finite codes, which are increasing in value. */
int orc_e4m3_encode(double v) {
  int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  int lo = 0, hi = 126; /* largest code with value <= a */
  if (a >= 448.0) return (neg << 7) | 126;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (orc_e4m3_value(mid) <= a) lo = mid; else hi = mid - 1;
  }
  int c = lo;
  if (c < 126) {
    double d0 = a - orc_e4m3_value(c), d1 = orc_e4m3_value(c + 1) - a;
    if (d1 < d0 || (d1 == d0 && (c & 1))) c = c + 1;
  }
  return (neg << 7) | c;
}

/* E8M0 scale byte of a block with absolute maximum amax: 127 + e, e the
 * smallest integer with amax <= 448 * 2^e (127 for amax == 0). */
int orc_ue8m0(double amax) {
  if (!(amax > 0.0)) return 127;
  int e;
  frexp(amax, &e);
  e -= 9; /* near the answer (floor(log2 amax) - 8); the loops make it exact */
  while (ldexp(448.0, e) < amax) ++e;
  while (e > -127 && ldexp(448.0, e - 1) >= amax) --e;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e + 127;
}

/* Quantise nrows rows of ncols (ncols % 32 == 0) values in blocks of 32 along
 * each row: scales[r, b] (E8M0 bytes), codes[r, c] (E4M3).  in_dtype: 0 f32,
 * 1 bf16, 2 f64. */
void orc_quant_rows(int64_t nrows, int ncols, int in_dtype, const void* in, uint8_t* codes,
                    uint8_t* scales) {
  /* rows are independent: spread over threads when there are many (inside another
   * parallel region this runs on the calling thread) */
#pragma omp parallel for schedule(static) if (nrows >= 256)
  for (int64_t r = 0; r < nrows; ++r)
    for (int b = 0; b < ncols / ORC_QB; ++b) {
      double v[ORC_QB], amax = 0.0;
      for (int i = 0; i < ORC_QB; ++i) {
        size_t idx = (size_t)r * ncols + (size_t)b * ORC_QB + i;
        v[i] = in_dtype == 2 ? ((const double*)in)[idx] : orc_load(in, idx, in_dtype);
        if (fabs(v[i]) > amax) amax = fabs(v[i]);
      }
      int s = orc_ue8m0(amax);
      scales[(size_t)r * (ncols / ORC_QB) + b] = (uint8_t)s;
      for (int i = 0; i < ORC_QB; ++i)
        codes[(size_t)r * ncols + (size_t)b * ORC_QB + i] =
            (uint8_t)orc_e4m3_encode(ldexp(v[i], 127 - s));
    }
}

static inline double orc_deq(const uint8_t* codes, const uint8_t* scales, size_t idx,
                             size_t sidx) {
  return ldexp(orc_e4m3_value(codes[idx]), (int)scales[sidx] - 127);
}

/* FP8 SwiGLU FFN of a set of rows.  Inputs are already quantised (codes +
 * scales): rows xq/xs [nrows, H] / [nrows, H/32]; per expert the weights
 * wg/wu [E, H, I] with scales [E, H/32, I] (blocks along H), wd [E, I, H]
 * with scales [E, I/32, H] (blocks along I).  g and u accumulate the
 * dequantised products in fp64; a = silu(g) * u is quantised per row in
 * blocks of 32 (orc_quant_rows rule) and dequantised before the down
 * projection; yp in fp64.  a_out (fp64, before quantisation), a_codes /
 * a_scales may be NULL. */
void orc_ffn_rows_fp8(int H, int I, int nrows, const int32_t* row_expert, const uint8_t* xq,
                      const uint8_t* xs, const uint8_t* wgq, const uint8_t* wgs,
                      const uint8_t* wuq, const uint8_t* wus, const uint8_t* wdq,
                      const uint8_t* wds, double* yp, double* a_out, uint8_t* a_codes,
                      uint8_t* a_scales, int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  const int HB = H / ORC_QB, IB = I / ORC_QB;
#pragma omp parallel
  {
    double* g = (double*)malloc(sizeof(double) * (size_t)I);
    double* u = (double*)malloc(sizeof(double) * (size_t)I);
    double* a = (double*)malloc(sizeof(double) * (size_t)I);
    uint8_t* aq = (uint8_t*)malloc((size_t)I);
    uint8_t* as = (uint8_t*)malloc((size_t)IB);
#pragma omp for schedule(dynamic, 1)
    for (int r = 0; r < nrows; ++r) {
      size_t e = (size_t)row_expert[r];
      for (int i = 0; i < I; ++i) g[i] = u[i] = 0.0;
      for (int h = 0; h < H; ++h) {
        double xv = orc_deq(xq, xs, (size_t)r * H + h, (size_t)r * HB + h / ORC_QB);
        for (int i = 0; i < I; ++i) {
          size_t wi = (e * H + h) * (size_t)I + i;
          size_t si = (e * HB + h / ORC_QB) * (size_t)I + i;
          g[i] += xv * orc_deq(wgq, wgs, wi, si);
          u[i] += xv * orc_deq(wuq, wus, wi, si);
        }
      }
      for (int i = 0; i < I; ++i) {
        a[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
        if (a_out) a_out[(size_t)r * I + i] = a[i];
      }
      orc_quant_rows(1, I, 2, a, aq, as);
      if (a_codes) memcpy(a_codes + (size_t)r * I, aq, (size_t)I);
      if (a_scales) memcpy(a_scales + (size_t)r * IB, as, (size_t)IB);
      double* y = yp + (size_t)r * H;
      for (int h = 0; h < H; ++h) y[h] = 0.0;
      for (int i = 0; i < I; ++i) {
        double av = orc_deq(aq, as, (size_t)i, (size_t)(i / ORC_QB));
        for (int h = 0; h < H; ++h) {
          size_t wi = (e * I + i) * (size_t)H + h;
          size_t si = (e * IB + i / ORC_QB) * (size_t)H + h;
          y[h] += av * orc_deq(wdq, wds, wi, si);
        }
      }
    }
    free(g);
    free(u);
    free(a);
    free(aq);
    free(as);
  }
}

/* Element-wise forms of the FP8 helpers (for the pins in tests/). */
void orc_e4m3_encode_vec(int64_t n, const double* v, uint8_t* codes) {
  for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)orc_e4m3_encode(v[i]);
}
void orc_e4m3_value_vec(int64_t n, const uint8_t* codes, double* v) {
  for (int64_t i = 0; i < n; ++i) v[i] = orc_e4m3_value(codes[i]);
}
void orc_ue8m0_vec(int64_t n, const double* amax, uint8_t* bytes) {
  for (int64_t i = 0; i < n; ++i) bytes[i] = (uint8_t)orc_ue8m0(amax[i]);
}
