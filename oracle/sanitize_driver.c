/*
 * sanitize_driver.c -- runs every function of bsa_oracle.c on small, ragged
 * inputs so that the oracle can be built and exercised under AddressSanitizer
 * and UndefinedBehaviorSanitizer (host code only).
 *
 * TEST INFRASTRUCTURE ONLY, like the oracle itself: built and run by the CPU
 * test suite (tests/test_oracle_sanitize.py), never by the product path.
 * Exit status 0 means every call returned and the few invariants checked
 * here held; the sanitizers abort the process on the first error they find.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_num_threads(void);
int oracle_radial_window(int64_t d, int64_t h0, int64_t beta, int64_t bk, int64_t* h_eff);
int64_t oracle_radial_count_pairs(int64_t T, int64_t Hs, int64_t Ws, int64_t h0, int64_t beta,
                                  int64_t bk);
void oracle_build_mask_radial(int64_t T, int64_t Hs, int64_t Ws, int64_t bq, int64_t bk,
                              int64_t h0, int64_t beta, uint8_t* mask);
int oracle_build_mask_pooled(int64_t B, int64_t H, int64_t N, int64_t D, int64_t bq, int64_t bk,
                             int dtype, const void* q, int64_t qsb, int64_t qsn, int64_t qsh,
                             const void* k, int64_t ksb, int64_t ksn, int64_t ksh, double scale,
                             int mode, double param, uint8_t* mask, double* scores_out,
                             double* margin_out, const double* levels_tau, int64_t n_levels);
int64_t oracle_compact(int64_t B, int64_t H, int64_t nQ, int64_t nK, const uint8_t* mask,
                       int64_t mask_head_stride, const uint8_t* skip, int32_t* row_ptr,
                       int32_t* kv_idx);
void oracle_order_lists(int64_t N, int64_t bq, int64_t bk, int64_t nQ, int64_t R, int order,
                        const int32_t* row_ptr, const int32_t* kv_in, int32_t* kv_out);
void oracle_make_permutation(int64_t T, int64_t Hs, int64_t Ws, int kind, const int64_t* axes,
                             int32_t* perm);
int oracle_choose_token_orders(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                               int64_t D, int64_t bq, int64_t bk, int dtype, const void* q,
                               const void* k, double scale, int mode, double param,
                               int32_t* order_out, int64_t* counts_out);
int oracle_pyramid_attention(int64_t B, int64_t H, int64_t N, int64_t D, int64_t bq, int64_t bk,
                             int dtype, const void* q, int64_t qsb, int64_t qsn, int64_t qsh,
                             const void* k, int64_t ksb, int64_t ksn, int64_t ksh,
                             const void* v, int64_t vsb, int64_t vsn, int64_t vsh,
                             double scale, const uint8_t* mask, int64_t mask_head_stride,
                             int64_t n_rows, const int64_t* rows, double* o_out,
                             double* lse_out);
void oracle_pyramid_regions(int64_t N, int64_t bk, int64_t n_levels, int64_t* region_block,
                            int64_t* region_rows);
int64_t oracle_compact_pyramid(int64_t B, int64_t H, int64_t nQ, int64_t nK, int64_t N,
                               int64_t bk, int64_t n_levels, const uint8_t* mask,
                               int64_t mask_head_stride, int32_t* row_ptr, int32_t* kv_idx,
                               uint8_t* kv_eighths);
int oracle_attention(int64_t B, int64_t H, int64_t N, int64_t D, int64_t bq, int64_t bk,
                     int dtype, const void* q, int64_t qsb, int64_t qsn, int64_t qsh,
                     const void* k, int64_t ksb, int64_t ksn, int64_t ksh, const void* v,
                     int64_t vsb, int64_t vsn, int64_t vsh, double scale, const uint8_t* mask,
                     int64_t mask_head_stride, int64_t n_rows, const int64_t* rows,
                     double* o_out, double* lse_out, double* gap_out, int order);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, enough for test inputs */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (double)((g_state * 2685821657736338717ull) >> 11) / 9007199254740992.0;
}

static int fails = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++fails;                                                     \
    }                                                              \
  } while (0)

/* One geometry: B x H heads of N = T*Hs*Ws tokens, head dim D. */
static void run_case(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws, int64_t D,
                     int64_t bq, int64_t bk) {
  const int64_t N = T * Hs * Ws, nQ = (N + bq - 1) / bq, nK = (N + bk - 1) / bk;
  const int64_t R = B * H * nQ, n = B * N * H * D;
  float* q = malloc(sizeof(float) * n);
  float* k = malloc(sizeof(float) * n);
  float* v = malloc(sizeof(float) * n);
  uint16_t* qb = malloc(sizeof(uint16_t) * n);
  for (int64_t i = 0; i < n; ++i) {
    q[i] = (float)(2.0 * uniform() - 1.0);
    k[i] = (float)(2.0 * uniform() - 1.0);
    v[i] = (float)(2.0 * uniform() - 1.0);
    uint32_t u;
    memcpy(&u, &q[i], 4);
    qb[i] = (uint16_t)(u >> 16);
  }
  const int64_t sb = N * H * D, sn = H * D, sh = D;

  /* radial */
  int64_t h;
  for (int64_t d = 0; d < 40; ++d) oracle_radial_window(d, 3 * bk, 2, bk, &h);
  uint8_t* rmask = malloc((size_t)(nQ * nK));
  oracle_build_mask_radial(T, Hs, Ws, bq, bk, bk, 2, rmask);
  if (N <= 600) CHECK(oracle_radial_count_pairs(T, Hs, Ws, bk, 2, bk) > 0);

  /* pooled: every mode, float and bf16 inputs */
  uint8_t* pmask = malloc((size_t)(R * nK));
  double* scores = malloc(sizeof(double) * R * nK);
  double* margin = malloc(sizeof(double) * R);
  const double taus[3] = {0.3, 0.6, 0.9};
  for (int mode = 0; mode <= 4; ++mode) {
    const double param = (mode == 0 || mode == 2) ? 2.0 : 0.5;
    CHECK(oracle_build_mask_pooled(B, H, N, D, bq, bk, 1, q, sb, sn, sh, k, sb, sn, sh, 0.3,
                                   mode, param, pmask, scores, margin,
                                   mode == 4 ? taus : NULL, mode == 4 ? 3 : 0) == 0);
  }
  CHECK(oracle_build_mask_pooled(B, H, N, D, bq, bk, 0, qb, sb, sn, sh, qb, sb, sn, sh, 0.3, 1,
                                 0.7, pmask, NULL, NULL, NULL, 0) == 0);

  /* compaction, with a skip set, and list orders */
  uint8_t* skip = malloc((size_t)(R * nK));
  for (int64_t i = 0; i < R * nK; ++i) skip[i] = uniform() < 0.3;
  int32_t* rp = malloc(sizeof(int32_t) * (R + 1));
  int32_t* kv = malloc(sizeof(int32_t) * (R * nK + 1));
  int32_t* kv2 = malloc(sizeof(int32_t) * (R * nK + 1));
  const int64_t nnz = oracle_compact(B, H, nQ, nK, pmask, nQ * nK, skip, rp, kv);
  CHECK(nnz == rp[R]);
  for (int order = 0; order <= 1; ++order) oracle_order_lists(N, bq, bk, nQ, R, order, rp, kv, kv2);

  /* attention with gaps in both orders, every row, fp32 and bf16 */
  int64_t* rows = malloc(sizeof(int64_t) * R);
  for (int64_t r = 0; r < R; ++r) rows[r] = r;
  double* o = malloc(sizeof(double) * R * bq * D);
  double* lse = malloc(sizeof(double) * R * bq);
  double* gap = malloc(sizeof(double) * R * nK);
  for (int order = 0; order <= 1; ++order)
    CHECK(oracle_attention(B, H, N, D, bq, bk, 1, q, sb, sn, sh, k, sb, sn, sh, v, sb, sn, sh,
                           0.2, pmask, nQ * nK, R, rows, o, lse, gap, order) == 0);
  CHECK(oracle_attention(B, H, N, D, bq, bk, 0, qb, sb, sn, sh, qb, sb, sn, sh, qb, sb, sn, sh,
                         0.2, rmask, 0, R, rows, o, lse, NULL, 0) == 0);

  /* per-head order choice over the six axis orders (both per-row modes) */
  {
    int32_t ord[8];
    int64_t cnt[8 * 6];
    if (H <= 8) {
      CHECK(oracle_choose_token_orders(B, H, T, Hs, Ws, D, bq, bk, 1, q, k, 0.3, 1, 0.5, ord,
                                       cnt) == 0);
      CHECK(oracle_choose_token_orders(B, H, T, Hs, Ws, D, bq, bk, 0, qb, qb, 0.3, 0, 2.0, ord,
                                       cnt) == 0);
      for (int64_t h = 0; h < H; ++h) CHECK(ord[h] >= 0 && ord[h] < 6);
    }
  }

  /* permutations: all axis orders and a few boxes */
  int32_t* perm = malloc(sizeof(int32_t) * N);
  const int64_t axes[6][3] = {{0, 1, 2}, {0, 2, 1}, {1, 0, 2}, {1, 2, 0}, {2, 0, 1}, {2, 1, 0}};
  for (int i = 0; i < 6; ++i) oracle_make_permutation(T, Hs, Ws, 0, axes[i], perm);
  const int64_t box[3] = {2, 3, 2};
  oracle_make_permutation(T, Hs, Ws, 1, box, perm);

  /* pyramid: regions, lists and attention on a level mask, three and four
     levels (N a multiple of 2^(levels-1)) */
  for (int64_t L = 3; L <= 4; ++L) {
    if (N % ((int64_t)1 << (L - 1)) != 0) continue;
    int64_t rb[5], rr[5];
    oracle_pyramid_regions(N, bk, L, rb, rr);
    uint8_t* lv = malloc((size_t)(R * nK));
    for (int64_t i = 0; i < R * nK; ++i) lv[i] = (uint8_t)(uniform() * (double)(L + 1));
    const int64_t nA = rb[L];
    int32_t* prp = malloc(sizeof(int32_t) * (R + 1));
    int32_t* pkv = malloc(sizeof(int32_t) * (R * nA + 1));
    uint8_t* pqm = malloc((size_t)(R * nA + 1));
    const int64_t pn = oracle_compact_pyramid(B, H, nQ, nK, N, bk, L, lv, nQ * nK, prp, pkv, pqm);
    CHECK(pn == prp[R]);
    CHECK(oracle_pyramid_attention(B, H, N, D, bq, bk, 1, q, sb, sn, sh, k, sb, sn, sh, v, sb,
                                   sn, sh, 0.2, lv, nQ * nK, R, rows, o, lse) == 0);
    free(lv); free(prp); free(pkv); free(pqm);
  }
  for (int64_t r = 0; r < R; ++r) {
    const int64_t len = ((r % nQ) + 1) * bq <= N ? bq : N - (r % nQ) * bq;
    for (int64_t i = 0; i < len; ++i) CHECK(!isnan(lse[r * bq + i]));
  }
  free(q); free(k); free(v); free(qb); free(rmask); free(pmask); free(scores); free(margin);
  free(skip); free(rp); free(kv); free(kv2); free(rows); free(o); free(lse); free(gap); free(perm);
}

int main(void) {
  printf("oracle threads: %d\n", oracle_num_threads());
  run_case(1, 2, 4, 8, 8, 16, 64, 64);   /* aligned blocks */
  run_case(2, 1, 5, 6, 7, 8, 16, 16);    /* ragged last blocks (N = 210) */
  run_case(1, 3, 3, 5, 9, 8, 32, 16);    /* ragged, Bq != Bk (N = 135, odd) */
  run_case(1, 1, 2, 4, 16, 8, 64, 64);   /* N = 128 */
  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("sanitized oracle run ok\n");
  return 0;
}
