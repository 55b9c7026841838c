/* Drives every function of the CPU oracle (oracle/moe_oracle.c, compiled into this program)
 * on small seeded inputs, for a build with AddressSanitizer and UndefinedBehaviorSanitizer:
 * any out-of-bounds access, use after free, leak, signed overflow, misaligned access or
 * invalid shift aborts the run.  It also checks the layout's invariants (every kept slot
 * exactly once, offsets the exclusive scan of counts) so that a run that stays in bounds
 * for the wrong reason fails too.  Test infrastructure only, like the oracle itself. */
#include "../../oracle/moe_oracle.c"

#include <stdio.h>

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) { /* SplitMix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static float uniform(void) { return (float)((next_u64() >> 40) * (1.0 / 16777216.0)) * 2.0f - 1.0f; }
static uint16_t bf16_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                   \
    }                                                             \
  } while (0)

static int run_case(int T, int E, int k, int H, int I, int C, int renorm, int ties) {
  const size_t tk = (size_t)T * k;
  float* logits = malloc(sizeof(float) * T * E);
  for (int i = 0; i < T * E; ++i)
    logits[i] = ties ? (float)(next_u64() % 3) : 3.0f * uniform();
  int32_t* ids = malloc(sizeof(int32_t) * tk);
  float* w = malloc(sizeof(float) * tk);
  uint8_t* keep = malloc(tk);
  orc_route(T, E, k, renorm, logits, ids, w);
  orc_capacity(T, E, k, C, ids, w, keep);
  int32_t* counts = malloc(sizeof(int32_t) * E);
  int32_t* offsets = malloc(sizeof(int32_t) * (E + 1));
  int32_t* row_token = malloc(sizeof(int32_t) * tk);
  int32_t* s2r = malloc(sizeof(int32_t) * tk);
  const int N = orc_layout(T, E, k, ids, keep, counts, offsets, row_token, s2r);
  /* invariants */
  CHECK(offsets[0] == 0 && offsets[E] == N);
  for (int e = 0; e < E; ++e) CHECK(offsets[e + 1] - offsets[e] == counts[e]);
  for (int e = 0; e < E; ++e) CHECK(C <= 0 || counts[e] <= C);
  int* seen = calloc((size_t)N + 1, sizeof(int));
  for (size_t s = 0; s < tk; ++s) {
    if (!keep[s]) {
      CHECK(s2r[s] == -1);
      continue;
    }
    CHECK(s2r[s] >= 0 && s2r[s] < N && row_token[s2r[s]] == (int)(s / k));
    seen[s2r[s]] += 1;
  }
  for (int r = 0; r < N; ++r) CHECK(seen[r] == 1);
  free(seen);

  /* grouped selection (2 groups, 1 taken when k fits in half the experts) */
  if (E % 2 == 0 && k <= E / 2) {
    int32_t* gids = malloc(sizeof(int32_t) * tk);
    float* gw = malloc(sizeof(float) * tk);
    orc_route_grouped(T, E, k, renorm, 2, 1, logits, gids, gw);
    free(gids);
    free(gw);
  }

  /* rows: bf16 and f32 FFN, gather, combine */
  uint16_t* x16 = malloc(sizeof(uint16_t) * T * H);
  float* x32 = malloc(sizeof(float) * T * H);
  for (int i = 0; i < T * H; ++i) {
    x32[i] = uniform();
    x16[i] = bf16_of(x32[i]);
  }
  const size_t wn = (size_t)E * H * I;
  uint16_t* wg = malloc(2 * wn);
  uint16_t* wu = malloc(2 * wn);
  uint16_t* wd = malloc(2 * wn);
  for (size_t i = 0; i < wn; ++i) {
    wg[i] = bf16_of(0.1f * uniform());
    wu[i] = bf16_of(0.1f * uniform());
    wd[i] = bf16_of(0.1f * uniform());
  }
  uint16_t* xp = malloc(sizeof(uint16_t) * ((size_t)N + 1) * H);
  orc_gather(N, H, 2, x16, row_token, xp);
  int32_t* rexp = malloc(sizeof(int32_t) * ((size_t)N + 1));
  for (int e = 0; e < E; ++e)
    for (int r = offsets[e]; r < offsets[e + 1]; ++r) rexp[r] = e;
  double* yp = malloc(sizeof(double) * ((size_t)N + 1) * H);
  double* a = malloc(sizeof(double) * ((size_t)N + 1) * I);
  orc_ffn_rows(H, I, ORC_BF16, ORC_BF16, N, rexp, xp, wg, wu, wd, yp, a, 2);
  int32_t* toks = malloc(sizeof(int32_t) * T);
  for (int t = 0; t < T; ++t) toks[t] = t;
  double* y = malloc(sizeof(double) * T * H);
  orc_combine(T, toks, H, k, w, s2r, yp, y);
  /* the f32 path on the same rows (f32 weights widened from the bf16 ones) */
  float* wg32 = malloc(4 * wn);
  float* wu32 = malloc(4 * wn);
  float* wd32 = malloc(4 * wn);
  for (size_t i = 0; i < wn; ++i) {
    uint32_t u;
    u = (uint32_t)wg[i] << 16; memcpy(&wg32[i], &u, 4);
    u = (uint32_t)wu[i] << 16; memcpy(&wu32[i], &u, 4);
    u = (uint32_t)wd[i] << 16; memcpy(&wd32[i], &u, 4);
  }
  float* xp32 = malloc(sizeof(float) * ((size_t)N + 1) * H);
  orc_gather(N, H, 4, x32, row_token, xp32);
  orc_ffn_rows(H, I, ORC_F32, ORC_F32, N, rexp, xp32, wg32, wu32, wd32, yp, NULL, 1);

  /* router logits from the hidden states */
  double* rl = malloc(sizeof(double) * T * E);
  orc_router_logits(T, H, E, ORC_BF16, x16, wg, rl);
  orc_router_logits(T, H, E, ORC_F32, x32, wg32, rl);

  /* FP8: rows and weights (blocks of 32 along the reduction dimension), the FFN */
  if (H % 32 == 0 && I % 32 == 0) {
    uint8_t* xq = malloc((size_t)N * H + 1);
    uint8_t* xs = malloc((size_t)N * H / 32 + 1);
    orc_quant_rows(N, H, ORC_BF16, xp, xq, xs);
    /* weights transposed to [E][N][K] rows, as the Python wrapper quantises them */
    uint8_t* gq = malloc(wn), *gs = malloc(wn / 32), *uq = malloc(wn), *us = malloc(wn / 32);
    uint8_t* dq = malloc(wn), *ds = malloc(wn / 32);
    uint16_t* tmp = malloc(2 * wn);
    for (int pass = 0; pass < 3; ++pass) {
      const uint16_t* src = pass == 0 ? wg : pass == 1 ? wu : wd;
      const int K = pass < 2 ? H : I, M = pass < 2 ? I : H;
      for (int e = 0; e < E; ++e)
        for (int kk = 0; kk < K; ++kk)
          for (int m = 0; m < M; ++m)
            tmp[((size_t)e * M + m) * K + kk] = src[((size_t)e * K + kk) * M + m];
      uint8_t* codes = malloc(wn);
      uint8_t* sc = malloc(wn / 32);
      orc_quant_rows((int64_t)E * M, K, ORC_BF16, tmp, codes, sc);
      uint8_t* q = pass == 0 ? gq : pass == 1 ? uq : dq;
      uint8_t* s = pass == 0 ? gs : pass == 1 ? us : ds;
      for (int e = 0; e < E; ++e)
        for (int kk = 0; kk < K; ++kk)
          for (int m = 0; m < M; ++m) {
            q[((size_t)e * K + kk) * M + m] = codes[((size_t)e * M + m) * K + kk];
            if (kk % 32 == 0)
              s[((size_t)e * (K / 32) + kk / 32) * M + m] = sc[((size_t)e * M + m) * (K / 32) + kk / 32];
          }
      free(codes);
      free(sc);
    }
    uint8_t* ac = malloc((size_t)N * I + 1);
    uint8_t* as = malloc((size_t)N * I / 32 + 1);
    orc_ffn_rows_fp8(H, I, N, rexp, xq, xs, gq, gs, uq, us, dq, ds, yp, a, ac, as, 2);
    free(xq); free(xs); free(gq); free(gs); free(uq); free(us); free(dq); free(ds);
    free(tmp); free(ac); free(as);
  }

  free(logits); free(ids); free(w); free(keep); free(counts); free(offsets);
  free(row_token); free(s2r); free(x16); free(x32); free(wg); free(wu); free(wd);
  free(xp); free(rexp); free(yp); free(a); free(toks); free(y); free(wg32); free(wu32);
  free(wd32); free(xp32); free(rl);
  return 0;
}

int main(void) {
  /* the specified exp over a sweep of its domain, and every E4M3 code and UE8M0 rule */
  for (float x = -90.0f; x <= 0.0f; x += 0.013f) (void)orc_exp(x);
  float worst;
  (void)orc_exp_max_ulp(-88.0f, -80.0f, &worst); /* about 1e6 values */
  for (int c = 0; c < 256; ++c) {
    const double v = orc_e4m3_value(c);
    if (v == v) CHECK((orc_e4m3_encode(v) & 0x7F) == (c & 0x7F) || v == 0.0);
  }
  for (int i = -40; i <= 40; ++i) (void)orc_ue8m0(ldexp(1.3, i));
  (void)orc_ue8m0(0.0);
  /* shapes: ragged, capped with ties, one expert, no renormalisation, k = E */
  if (run_case(37, 8, 2, 64, 96, 0, 1, 0)) return 1;
  if (run_case(50, 6, 3, 32, 64, 7, 1, 1)) return 1;
  if (run_case(9, 1, 1, 32, 32, 0, 1, 0)) return 1;
  if (run_case(20, 16, 4, 64, 32, 3, 0, 0)) return 1;
  if (run_case(5, 4, 4, 32, 64, 2, 1, 1)) return 1;
  printf("oracle driver ok\n");
  return 0;
}
