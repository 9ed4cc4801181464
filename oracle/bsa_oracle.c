/*
 * bsa_oracle.c -- plain, slow fp64 CPU oracle for block-sparse video attention.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it. It shares no code, header, table or helper
 * with the HIP library; the two meet only in the seeded inputs.
 *
 * Arithmetic: IEEE fp64, plain loops in the order written, compiled with
 * -ffp-contract=off and no fast-math. OpenMP splits independent rows only.
 *
 * Pages cited (titles of the web pages that describe the method):
 *   [Lite]   LiteAttention summary page (arXiv:2511.11062), numbered sections.
 *   [VMoBA]  VMoBA summary page (arXiv:2506.23858), numbered sections.
 *   [Radial] "MIT实验室推出Radial Attention：让视频AI生成快如闪电的神奇技术"
 *            (arXiv:2506.19852), paragraphs on energy decay, the static map
 *            and the O(n log n) complexity.
 *   [PARO]   PAROAttention summary page (arXiv:2506.16054), numbered sections.
 *   [PSA]    "浙江大学突破视频AI瓶颈:金字塔方法提升视频AI效率10倍"
 *            (arXiv:2512.04025), paragraphs on block-sparse keep/drop and
 *            average pooling.
 *
 * Geometry convention (the pages say only that the 3D video is flattened to
 * 1D; [PARO] section 二, [VMoBA] section 三): token i <-> (t, y, x) with
 * i = (t*Hs + y)*Ws + x; frame t(i) = i / F, in-frame position s(i) = i % F,
 * F = Hs*Ws. Row block a covers [a*Bq, min(N, (a+1)*Bq)), column block c
 * covers [c*Bk, min(N, (c+1)*Bk)); ragged last blocks keep their true sizes.
 *
 * Element types of input tensors: 0 = bf16 (uint16 bit patterns),
 * 1 = fp32, 2 = fp64. Widening to fp64 is exact.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_BF16 0
#define ORACLE_F32 1
#define ORACLE_F64 2

/* Threads the OpenMP loops below run on (reported with timings). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

static double widen(const void* base, int dtype, int64_t off) {
  if (dtype == ORACLE_BF16) {
    uint32_t u = ((uint32_t)((const uint16_t*)base)[off]) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
  }
  if (dtype == ORACLE_F32) return (double)((const float*)base)[off];
  return ((const double*)base)[off];
}

/* ------------------------------------------------------------------------ */
/* Radial window ([Radial]: attention weakens with spatial and temporal     */
/* distance; each frame mostly attends to its nearest frames and the weight */
/* falls off with frame distance by a fixed rule; the map is fixed ahead of */
/* time; total cost grows as n log n).                                      */
/*                                                                          */
/* Reading taken: frame distance d falls in band r(d) = number of base-beta */
/* digits of d (r(0) = 0). The spatial half-width halves per band:          */
/* h_r = floor(h0 / beta^r). Once h_r would drop below half a key block     */
/* (h_min = Bk/2), the window stays at h_min and instead only every         */
/* beta^(r - r*)-th distance of band r is kept, r* = last band with         */
/* h_r >= h_min. Token pair (i, j) is kept iff its distance is kept and     */
/* |s(i) - s(j)| < h_eff(d).                                                */
/* Returns 1 if distance d is kept and writes its half-width.               */
/* ------------------------------------------------------------------------ */
int oracle_radial_window(int64_t d, int64_t h0, int64_t beta, int64_t bk,
                         int64_t* h_eff) {
  int64_t r = 0, p = 1; /* p = beta^r(d) */
  while (p <= d) { p *= beta; ++r; }
  int64_t h_min = bk / 2;
  /* r* = max{ r : floor(h0 / beta^r) >= h_min } */
  int64_t rstar = 0, q = 1;
  while (h0 / (q * beta) >= h_min) { q *= beta; ++rstar; }
  if (r <= rstar) {
    int64_t br = 1;
    for (int64_t k = 0; k < r; ++k) br *= beta;
    *h_eff = h0 / br;
    return 1;
  }
  int64_t step = 1;
  for (int64_t k = 0; k < r - rstar; ++k) step *= beta;
  *h_eff = h_min;
  return (d % step) == 0;
}

/* Brute-force count of kept token pairs (tiny grids only). */
int64_t oracle_radial_count_pairs(int64_t T, int64_t Hs, int64_t Ws, int64_t h0,
                                  int64_t beta, int64_t bk) {
  int64_t F = Hs * Ws, N = T * F, cnt = 0;
  for (int64_t i = 0; i < N; ++i)
    for (int64_t j = 0; j < N; ++j) {
      int64_t ti = i / F, tj = j / F, h;
      int64_t d = ti > tj ? ti - tj : tj - ti;
      if (!oracle_radial_window(d, h0, beta, bk, &h)) continue;
      int64_t ds = (i % F) - (j % F);
      if (ds < 0) ds = -ds;
      if (ds < h) ++cnt;
    }
  return cnt;
}

/* Tile rule (binary keep/drop of whole blocks, [PSA]): tile (a, c) is kept
 * iff some query token of row block a and some key token of column block c
 * form a kept pair. For each query token the check is: in every frame that
 * column block c touches, is there a key of the block whose in-frame position
 * lies within the window of that frame distance. mask is [nQ][nK], head- and
 * batch-independent. */
void oracle_build_mask_radial(int64_t T, int64_t Hs, int64_t Ws, int64_t bq,
                              int64_t bk, int64_t h0, int64_t beta,
                              uint8_t* mask) {
  int64_t F = Hs * Ws, N = T * F;
  int64_t nQ = (N + bq - 1) / bq, nK = (N + bk - 1) / bk;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t a = 0; a < nQ; ++a) {
    int64_t i0 = a * bq, i1 = (a + 1) * bq < N ? (a + 1) * bq : N;
    for (int64_t c = 0; c < nK; ++c) {
      int64_t j0 = c * bk, j1 = (c + 1) * bk < N ? (c + 1) * bk : N;
      int keep = 0;
      for (int64_t i = i0; i < i1 && !keep; ++i) {
        int64_t ti = i / F, si = i % F;
        for (int64_t tk = j0 / F; tk <= (j1 - 1) / F && !keep; ++tk) {
          int64_t d = ti > tk ? ti - tk : tk - ti, h;
          if (!oracle_radial_window(d, h0, beta, bk, &h)) continue;
          /* keys of block c inside frame tk: in-frame positions [lo, hi] */
          int64_t lo = (j0 > tk * F ? j0 : tk * F) - tk * F;
          int64_t hi = ((j1 < (tk + 1) * F ? j1 : (tk + 1) * F) - 1) - tk * F;
          int64_t dist = 0;
          if (si < lo) dist = lo - si;
          else if (si > hi) dist = si - hi;
          if (dist < h) keep = 1;
        }
      }
      mask[a * nK + c] = (uint8_t)keep;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Pooled block selection ([PSA]: keys are mean-pooled block by block;       */
/* [VMoBA] sections 三 and 六: block relevance from pooled scores, number of */
/* blocks per query set by a threshold that follows how concentrated the    */
/* attention is; [PSA] ablation: threshold allocation beats quantiles).     */
/*                                                                          */
/* Steps, per (b, h):                                                       */
/* 1. qbar_a = (sum over i in row block a of q_i, ascending i) / |R_a|;     */
/*    kbar_c likewise over column block c.                                  */
/* 2. S_ac = scale * (sum_k qbar_ak * kbar_ck), k ascending, each product   */
/*    and sum rounded separately, then one multiply by scale.               */
/* 3. Row a: order c by (S desc, c asc).                                    */
/* 4. mode 0 (top-k): keep the first min(k, nK) of that order.              */
/*    mode 1 (cumulative mass): e_c = exp(S_ac - max_c S_ac); Z = sum of e  */
/*    in ascending c; p_c = e_c / Z; walk the order accumulating p and keep  */
/*    the shortest prefix whose running sum is >= tau_p (all if never).     */
/* margin_out[row] (optional) = distance of the running sum from tau_p at   */
/* the last step inside the prefix and the step before it (mode 1).         */
/*                                                                          */
/* Global modes ([VMoBA] section 三: rank the relevance of every query with */
/* every block and serve the strongest combinations first, instead of the   */
/* same number of blocks per query; the number of blocks a head keeps       */
/* follows how concentrated its attention is). Per (b, h), all nQ*nK pairs  */
/* are ordered together by (key desc, a*nK + c asc) and                     */
/*    mode 2 (global top-k): the first min(k, nQ*nK) pairs are kept, key S; */
/*    mode 3 (global cumulative mass): key p_ac = e_ac / Z_a with e and Z   */
/*      of row a as in mode 1; the shortest prefix whose running sum of p   */
/*      reaches tau_p * nQ is kept (all pairs if never, or if tau_p = 1).   */
/* Pyramid levels (mode 4; [PSA]: each query-block/key-block pair gets a    */
/* resolution level by its importance, with thresholds rather than          */
/* quantiles): row a walks its blocks in (S desc, c asc) order accumulating */
/* the mode-1 softmax mass; a block whose running sum (including itself)    */
/* first reaches levels_tau[l] or is still below it joins level l, for      */
/* l = 0 .. n_levels-1 with levels_tau non-decreasing; later blocks are     */
/* dropped. mask = 1 + level (0 = dropped). The row's first block is always */
/* at level 0.                                                              */
/* In both, every row also keeps its own first block in (S desc, c asc)     */
/* order, so that no row is left empty. margin_out[bh*nQ] holds the head's  */
/* margin for mode 3 (as in mode 1, against tau_p * nQ); other rows inf.    */
/* ------------------------------------------------------------------------ */
typedef struct { double s; int64_t c; } scored;

static int cmp_scored(const void* x, const void* y) {
  const scored* a = (const scored*)x;
  const scored* b = (const scored*)y;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->c > b->c) - (a->c < b->c);
}

int oracle_build_mask_pooled(int64_t B, int64_t H, int64_t N, int64_t D,
                             int64_t bq, int64_t bk, int dtype,
                             const void* q, int64_t qsb, int64_t qsn, int64_t qsh,
                             const void* k, int64_t ksb, int64_t ksn, int64_t ksh,
                             double scale, int mode, double param,
                             uint8_t* mask, double* scores_out,
                             double* margin_out, const double* levels_tau,
                             int64_t n_levels) {
  int64_t nQ = (N + bq - 1) / bq, nK = (N + bk - 1) / bk;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * H; ++bh) {
    int64_t b = bh / H, h = bh % H;
    double* qbar = (double*)malloc(sizeof(double) * nQ * D);
    double* kbar = (double*)malloc(sizeof(double) * nK * D);
    double* S = (double*)malloc(sizeof(double) * nQ * nK);
    scored* ord = (scored*)malloc(sizeof(scored) * nK);
    double* P = mode == 3 ? (double*)malloc(sizeof(double) * nQ * nK) : NULL;
    int global = mode == 2 || mode == 3;
    scored* gord = global ? (scored*)malloc(sizeof(scored) * nQ * nK) : NULL;
    if (!qbar || !kbar || !S || !ord || (mode == 3 && !P) || (global && !gord)) {
#pragma omp atomic write
      bad = 1;
      free(qbar); free(kbar); free(S); free(ord); free(P); free(gord);
      continue;
    }
    for (int64_t a = 0; a < nQ; ++a) {
      int64_t i0 = a * bq, i1 = (a + 1) * bq < N ? (a + 1) * bq : N;
      for (int64_t x = 0; x < D; ++x) {
        double acc = 0.0;
        for (int64_t i = i0; i < i1; ++i)
          acc = acc + widen(q, dtype, b * qsb + i * qsn + h * qsh + x);
        qbar[a * D + x] = acc / (double)(i1 - i0);
      }
    }
    for (int64_t c = 0; c < nK; ++c) {
      int64_t j0 = c * bk, j1 = (c + 1) * bk < N ? (c + 1) * bk : N;
      for (int64_t x = 0; x < D; ++x) {
        double acc = 0.0;
        for (int64_t j = j0; j < j1; ++j)
          acc = acc + widen(k, dtype, b * ksb + j * ksn + h * ksh + x);
        kbar[c * D + x] = acc / (double)(j1 - j0);
      }
    }
    for (int64_t a = 0; a < nQ; ++a) {
      int64_t row = bh * nQ + a;
      for (int64_t c = 0; c < nK; ++c) {
        double acc = 0.0;
        for (int64_t x = 0; x < D; ++x) {
          double pr = qbar[a * D + x] * kbar[c * D + x];
          acc = acc + pr;
        }
        S[a * nK + c] = scale * acc;
        if (scores_out) scores_out[row * nK + c] = S[a * nK + c];
      }
    }
    memset(mask + bh * nQ * nK, 0, (size_t)(nQ * nK));
    for (int64_t a = 0; a < nQ; ++a) {
      int64_t row = bh * nQ + a;
      for (int64_t c = 0; c < nK; ++c) {
        ord[c].s = S[a * nK + c];
        ord[c].c = c;
      }
      qsort(ord, (size_t)nK, sizeof(scored), cmp_scored);
      uint8_t* m = mask + row * nK;
      int64_t keep = nK;
      double margin = INFINITY;
      if (mode == 0) {
        keep = (int64_t)param < nK ? (int64_t)param : nK;
      } else if (mode == 1) {
        double smax = ord[0].s, Z = 0.0;
        for (int64_t c = 0; c < nK; ++c) Z = Z + exp(S[a * nK + c] - smax);
        double run = 0.0, prev = 0.0;
        keep = nK;
        for (int64_t t = 0; t < nK; ++t) {
          prev = run;
          run = run + exp(ord[t].s - smax) / Z;
          if (run >= param) { keep = t + 1; break; }
        }
        margin = fabs(run - param);
        if (keep > 1 && fabs(param - prev) < margin) margin = fabs(param - prev);
      } else if (mode == 4) {
        double smax = ord[0].s, Z = 0.0;
        for (int64_t c = 0; c < nK; ++c) Z = Z + exp(S[a * nK + c] - smax);
        double run = 0.0;
        int64_t lvl = 0;
        for (int64_t t = 0; t < nK && lvl < n_levels; ++t) {
          m[ord[t].c] = (uint8_t)(1 + lvl);
          run = run + exp(ord[t].s - smax) / Z;
          while (lvl < n_levels && run >= levels_tau[lvl]) ++lvl;
        }
        keep = 0; /* levels written above */
      } else {
        /* global modes: the row keeps its best block; p of the row for mode 3 */
        keep = 1;
        if (mode == 3) {
          double smax = ord[0].s, Z = 0.0;
          for (int64_t c = 0; c < nK; ++c) Z = Z + exp(S[a * nK + c] - smax);
          for (int64_t c = 0; c < nK; ++c) P[a * nK + c] = exp(S[a * nK + c] - smax) / Z;
        }
      }
      for (int64_t t = 0; t < keep; ++t) m[ord[t].c] = 1;
      if (margin_out) margin_out[row] = margin;
    }
    if (global) {
      int64_t n = nQ * nK;
      for (int64_t u = 0; u < n; ++u) {
        gord[u].s = mode == 2 ? S[u] : P[u];
        gord[u].c = u;
      }
      qsort(gord, (size_t)n, sizeof(scored), cmp_scored);
      int64_t keep = n;
      double margin = INFINITY;
      if (mode == 2) {
        keep = (int64_t)param < n ? (int64_t)param : n;
      } else if (param >= 1.0) {
        keep = n; /* the whole mass: every pair, however the sum rounds */
      } else {
        double target = param * (double)nQ, run = 0.0, prev = 0.0;
        for (int64_t t = 0; t < n; ++t) {
          prev = run;
          run = run + gord[t].s;
          if (run >= target) { keep = t + 1; break; }
        }
        margin = fabs(run - target);
        if (keep > 1 && fabs(target - prev) < margin) margin = fabs(target - prev);
      }
      for (int64_t t = 0; t < keep; ++t) mask[bh * n + gord[t].c] = 1;
      if (margin_out) margin_out[bh * nQ] = margin;
    }
    free(qbar); free(kbar); free(S); free(ord); free(P); free(gord);
  }
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Compaction ([Lite] sections 三 and 六: a skipped tile must cost no memory */
/* transfer, so the loader walks only the kept tiles of each query block).   */
/* Row r = (b*H + h)*nQ + a; element (r, c) of the mask lives at            */
/* mask[(b*H + h)*mask_head_stride + a*nK + c] (stride 0: one mask for all  */
/* heads). kv_idx lists, per row, the ascending c with mask = 1 and         */
/* skip = 0; row_ptr is the exclusive prefix sum of the row lengths.        */
/* Returns nnz.                                                             */
/* ------------------------------------------------------------------------ */
int64_t oracle_compact(int64_t B, int64_t H, int64_t nQ, int64_t nK,
                       const uint8_t* mask, int64_t mask_head_stride,
                       const uint8_t* skip, int32_t* row_ptr, int32_t* kv_idx) {
  int64_t nnz = 0;
  for (int64_t bh = 0; bh < B * H; ++bh)
    for (int64_t a = 0; a < nQ; ++a) {
      int64_t r = bh * nQ + a;
      if (row_ptr) row_ptr[r] = (int32_t)nnz;
      for (int64_t c = 0; c < nK; ++c) {
        int on = mask[bh * mask_head_stride + a * nK + c] != 0;
        if (skip && skip[r * nK + c]) on = 0;
        if (on) {
          if (kv_idx) kv_idx[nnz] = (int32_t)c;
          ++nnz;
        }
      }
    }
  if (row_ptr) row_ptr[B * H * nQ] = (int32_t)nnz;
  return nnz;
}

/* ------------------------------------------------------------------------ */
/* Visiting order of the kept key blocks of a row ([Lite] section 五: a      */
/* radial-centric order of the blocks reaches the row's maximum sooner, so   */
/* the running-maximum test can skip more; section 十 expects more sparsity */
/* from a better order).                                                    */
/* Reading taken: blocks are visited by increasing distance between the     */
/* token midpoints of the key block and of the row block, ties to the lower */
/* block index. In integers, with the true (ragged) block bounds:           */
/*   cq2(a) = a*bq + min(N, (a+1)*bq) - 1   (twice the row-block midpoint)  */
/*   ck2(c) = c*bk + min(N, (c+1)*bk) - 1   (twice the key-block midpoint)  */
/*   key(c) = (|ck2(c) - cq2(a)|, c), ascending.                            */
/* order 0 keeps the ascending order. Lists are CSR rows r (R of them);     */
/* row r belongs to row block a = r % nQ.                                   */
/* ------------------------------------------------------------------------ */
static int64_t block_mid2(int64_t c, int64_t bk, int64_t N) {
  int64_t e = (c + 1) * bk < N ? (c + 1) * bk : N;
  return c * bk + e - 1;
}

/* 1 if key block x comes before key block y around twice-midpoint cq2. */
static int radial_before(int32_t x, int32_t y, int64_t cq2, int64_t bk, int64_t N) {
  int64_t dx = llabs(block_mid2(x, bk, N) - cq2);
  int64_t dy = llabs(block_mid2(y, bk, N) - cq2);
  return dx < dy || (dx == dy && x < y);
}

/* Insertion sort of n key blocks into radial-centric order. */
static void radial_sort(int32_t* v, int64_t n, int64_t cq2, int64_t bk, int64_t N) {
  for (int64_t i = 1; i < n; ++i) {
    int32_t x = v[i];
    int64_t j = i;
    while (j > 0 && radial_before(x, v[j - 1], cq2, bk, N)) {
      v[j] = v[j - 1];
      --j;
    }
    v[j] = x;
  }
}

void oracle_order_lists(int64_t N, int64_t bq, int64_t bk, int64_t nQ, int64_t R,
                        int order, const int32_t* row_ptr, const int32_t* kv_in,
                        int32_t* kv_out) {
  for (int64_t r = 0; r < R; ++r) {
    int64_t e0 = row_ptr[r], e1 = row_ptr[r + 1];
    for (int64_t e = e0; e < e1; ++e) kv_out[e] = kv_in[e];
    if (order == 1) radial_sort(kv_out + e0, e1 - e0, block_mid2(r % nQ, bq, N), bk, N);
  }
}

/* ------------------------------------------------------------------------ */
/* Token orders before blocking. [PARO] section 二: flattening the video to  */
/* one sequence scatters tokens that attend to each other; reordering them  */
/* (one of the 6 orders of the frame, height and width axes, chosen per     */
/* head) gathers them into block-shaped patterns. [VMoBA] section 三: blocks */
/* made of temporal chunks (about 3 frames), spatial patches, or            */
/* spatio-temporal cubes, cycled across layers.                             */
/* perm[i'] = original token index of new position i' (i = (t*Hs + y)*Ws+x).*/
/* kind 0: axis order; axes[0..2] name the slowest, middle and fastest axis */
/*         (0 = frame t, 1 = row y, 2 = column x).                          */
/* kind 1: box partition: boxes of axes[0] frames x axes[1] rows x axes[2]  */
/*         columns (smaller at the far edges), boxes in (t, y, x) order and */
/*         tokens inside a box in (t, y, x) order. Boxes of one frame's     */
/*         whole plane are temporal chunks, boxes of one frame are spatial  */
/*         patches, boxes spanning several frames are cubes.                */
/* Plain enumeration in the stated order.                                   */
/* ------------------------------------------------------------------------ */
void oracle_make_permutation(int64_t T, int64_t Hs, int64_t Ws, int kind,
                             const int64_t* axes, int32_t* perm) {
  int64_t n = 0;
  if (kind == 0) {
    int64_t ext[3] = {T, Hs, Ws};
    int64_t co[3];
    for (co[axes[0]] = 0; co[axes[0]] < ext[axes[0]]; ++co[axes[0]])
      for (co[axes[1]] = 0; co[axes[1]] < ext[axes[1]]; ++co[axes[1]])
        for (co[axes[2]] = 0; co[axes[2]] < ext[axes[2]]; ++co[axes[2]])
          perm[n++] = (int32_t)((co[0] * Hs + co[1]) * Ws + co[2]);
    return;
  }
  int64_t ct = axes[0], cy = axes[1], cx = axes[2];
  for (int64_t t0 = 0; t0 < T; t0 += ct)
    for (int64_t y0 = 0; y0 < Hs; y0 += cy)
      for (int64_t x0 = 0; x0 < Ws; x0 += cx)
        for (int64_t t = t0; t < t0 + ct && t < T; ++t)
          for (int64_t y = y0; y < y0 + cy && y < Hs; ++y)
            for (int64_t x = x0; x < x0 + cx && x < Ws; ++x)
              perm[n++] = (int32_t)((t * Hs + y) * Ws + x);
}

/* ------------------------------------------------------------------------ */
/* Per-head order choice ([PARO] section 二: a head takes, among the six    */
/* axis orders, the one under which its attention is most sparsity-        */
/* friendly; the pages give no formula, and the quantization side of the   */
/* choice is out of scope here). Reading: order o (axis orders in           */
/* lexicographic order, 0 = (0,1,2) ... 5 = (2,1,0)) scores, for head h,    */
/* the number of tiles oracle_build_mask_pooled (mode 0 or 1, param) keeps  */
/* for that head over the batch once Q and K are gathered into order o;     */
/* the head takes the fewest, ties to the lower order. q, k contiguous      */
/* [B][N][H][D] of dtype (0 bf16 bits, 1 float). counts_out [H][6].         */
/* Returns 0, or -1 on a bad argument or allocation failure.               */
/* ------------------------------------------------------------------------ */
int oracle_choose_token_orders(int64_t B, int64_t H, int64_t T, int64_t Hs, int64_t Ws,
                               int64_t D, int64_t bq, int64_t bk, int dtype, const void* q,
                               const void* k, double scale, int mode, double param,
                               int32_t* order_out, int64_t* counts_out) {
  static const int64_t axes[6][3] = {{0, 1, 2}, {0, 2, 1}, {1, 0, 2},
                                     {1, 2, 0}, {2, 0, 1}, {2, 1, 0}};
  if ((mode != 0 && mode != 1) || (dtype != 0 && dtype != 1)) return -1;
  const int64_t N = T * Hs * Ws, nQ = (N + bq - 1) / bq, nK = (N + bk - 1) / bk;
  const size_t esz = dtype == 0 ? 2 : 4, row = (size_t)D * esz;
  int32_t* perm = malloc(sizeof(int32_t) * (size_t)(N > 0 ? N : 1));
  char* qp = malloc((size_t)(B * N * H) * row + 1);
  char* kp = malloc((size_t)(B * N * H) * row + 1);
  uint8_t* mask = malloc((size_t)(B * H * nQ * nK) + 1);
  int bad = !perm || !qp || !kp || !mask;
  for (int64_t i = 0; i < H * 6; ++i) counts_out[i] = 0;
  for (int o = 0; o < 6 && !bad; ++o) {
    oracle_make_permutation(T, Hs, Ws, 0, axes[o], perm);
    /* gather: new position i' holds original token perm[i'] */
    for (int64_t b = 0; b < B; ++b)
      for (int64_t i = 0; i < N; ++i)
        for (int64_t h = 0; h < H; ++h) {
          const size_t dst = (size_t)((b * N + i) * H + h) * row;
          const size_t src = (size_t)((b * N + perm[i]) * H + h) * row;
          memcpy(qp + dst, (const char*)q + src, row);
          memcpy(kp + dst, (const char*)k + src, row);
        }
    if (oracle_build_mask_pooled(B, H, N, D, bq, bk, dtype, qp, N * H * D, H * D, D, kp,
                                 N * H * D, H * D, D, scale, mode, param, mask, NULL, NULL,
                                 NULL, 0) != 0) {
      bad = 1;
      break;
    }
    for (int64_t b = 0; b < B; ++b)
      for (int64_t h = 0; h < H; ++h) {
        const uint8_t* m = mask + (b * H + h) * nQ * nK;
        int64_t n = 0;
        for (int64_t e = 0; e < nQ * nK; ++e) n += m[e] != 0;
        counts_out[h * 6 + o] += n;
      }
  }
  for (int64_t h = 0; h < H && !bad; ++h) {
    int best = 0;
    for (int o = 1; o < 6; ++o)
      if (counts_out[h * 6 + o] < counts_out[h * 6 + best]) best = o;
    order_out[h] = best;
  }
  free(perm); free(qp); free(kp); free(mask);
  return bad ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Pyramid attention ([PSA]: key/value blocks kept at several resolutions,  */
/* each coarser level the average of the finer one; each pair of query and */
/* key block attends at its assigned level; the probabilities stay          */
/* consistent across levels).                                               */
/* Reading: level l of key block c holds bk / 2^l pooled keys, each the     */
/* mean of 2^l consecutive tokens of K (and of V); a pooled key stands for  */
/* its 2^l tokens, so its weight is 2^l exp(s): its score gets + l ln 2.    */
/* With equal scores inside every group the result equals level 0. N must  */
/* be a multiple of 2^l for the levels used. For query i of row block a,    */
/* the keys are: the tokens of blocks with mask = 1 (level 0) and the       */
/* pooled keys of blocks with mask = 1 + l; softmax over all of them.       */
/* Outputs as in oracle_attention (rows requested; NaN padding).            */
/* ------------------------------------------------------------------------ */
int oracle_pyramid_attention(int64_t B, int64_t H, int64_t N, int64_t D, int64_t bq,
                             int64_t bk, int dtype,
                             const void* q, int64_t qsb, int64_t qsn, int64_t qsh,
                             const void* k, int64_t ksb, int64_t ksn, int64_t ksh,
                             const void* v, int64_t vsb, int64_t vsn, int64_t vsh,
                             double scale, const uint8_t* mask, int64_t mask_head_stride,
                             int64_t n_rows, const int64_t* rows,
                             double* o_out, double* lse_out) {
  int64_t nQ = (N + bq - 1) / bq, nK = (N + bk - 1) / bk;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < n_rows; ++t) {
    int64_t row = rows[t];
    int64_t bh = row / nQ, a = row % nQ, b = bh / H, h = bh % H;
    int64_t i0 = a * bq, i1 = (a + 1) * bq < N ? (a + 1) * bq : N;
    const uint8_t* m = mask + bh * mask_head_stride + a * nK;
    /* the row's keys: (pooled) key vectors, value vectors, log-weights */
    int64_t nkeys = 0;
    for (int64_t c = 0; c < nK; ++c) {
      if (!m[c]) continue;
      int64_t len = ((c + 1) * bk < N ? (c + 1) * bk : N) - c * bk;
      nkeys += len >> (m[c] - 1);
    }
    double* kk = (double*)malloc(sizeof(double) * (nkeys > 0 ? nkeys : 1) * D);
    double* vv = (double*)malloc(sizeof(double) * (nkeys > 0 ? nkeys : 1) * D);
    double* lw = (double*)malloc(sizeof(double) * (nkeys > 0 ? nkeys : 1));
    double* sc = (double*)malloc(sizeof(double) * (nkeys > 0 ? nkeys : 1));
    double* qi = (double*)malloc(sizeof(double) * D);
    double* acc = (double*)malloc(sizeof(double) * D);
    if (!kk || !vv || !lw || !sc || !qi || !acc) {
#pragma omp atomic write
      bad = 1;
      free(kk); free(vv); free(lw); free(sc); free(qi); free(acc);
      continue;
    }
    int64_t u = 0;
    for (int64_t c = 0; c < nK; ++c) {
      if (!m[c]) continue;
      int64_t lev = m[c] - 1, g = (int64_t)1 << lev;
      int64_t j0 = c * bk, j1 = (c + 1) * bk < N ? (c + 1) * bk : N;
      for (int64_t j = j0; j < j1; j += g, ++u) {
        for (int64_t x = 0; x < D; ++x) {
          double sk = 0.0, sv = 0.0;
          for (int64_t jj = j; jj < j + g; ++jj) {
            sk = sk + widen(k, dtype, b * ksb + jj * ksn + h * ksh + x);
            sv = sv + widen(v, dtype, b * vsb + jj * vsn + h * vsh + x);
          }
          kk[u * D + x] = sk / (double)g;
          vv[u * D + x] = sv / (double)g;
        }
        lw[u] = log((double)g);
      }
    }
    for (int64_t r = 0; r < bq; ++r) {
      if (o_out) for (int64_t x = 0; x < D; ++x) o_out[(t * bq + r) * D + x] = NAN;
      if (lse_out) lse_out[t * bq + r] = NAN;
    }
    for (int64_t i = i0; i < i1; ++i) {
      int64_t r = i - i0;
      if (nkeys == 0) {
        if (o_out) for (int64_t x = 0; x < D; ++x) o_out[(t * bq + r) * D + x] = 0.0;
        if (lse_out) lse_out[t * bq + r] = -INFINITY;
        continue;
      }
      for (int64_t x = 0; x < D; ++x) qi[x] = widen(q, dtype, b * qsb + i * qsn + h * qsh + x);
      double mi = -INFINITY;
      for (int64_t w = 0; w < nkeys; ++w) {
        double dot = 0.0;
        for (int64_t x = 0; x < D; ++x) dot = dot + qi[x] * kk[w * D + x];
        sc[w] = scale * dot + lw[w];
        if (sc[w] > mi) mi = sc[w];
      }
      double li = 0.0;
      for (int64_t x = 0; x < D; ++x) acc[x] = 0.0;
      for (int64_t w = 0; w < nkeys; ++w) {
        double p = exp(sc[w] - mi);
        li = li + p;
        for (int64_t x = 0; x < D; ++x) acc[x] = acc[x] + p * vv[w * D + x];
      }
      if (o_out) for (int64_t x = 0; x < D; ++x) o_out[(t * bq + r) * D + x] = acc[x] / li;
      if (lse_out) lse_out[t * bq + r] = mi + log(li);
    }
    free(kk); free(vv); free(lw); free(sc); free(qi); free(acc);
  }
  return bad ? -1 : 0;
}

/* Rows of the level-l region of the augmented key array: level l holds     */
/* N / 2^l pooled rows, each region padded to a multiple of bk rows, levels */
/* in order. region_block[l] = first block of region l.                     */
void oracle_pyramid_regions(int64_t N, int64_t bk, int64_t n_levels, int64_t* region_block,
                            int64_t* region_rows) {
  int64_t blk = 0;
  for (int64_t l = 0; l < n_levels; ++l) {
    region_block[l] = blk;
    region_rows[l] = N >> l;
    blk += ((N >> l) + bk - 1) / bk;
  }
  region_block[n_levels] = blk;
}

/* Lists of augmented tiles for a pyramid mask ([PSA]: the logical block    */
/* size is decoupled from the hardware tile). Logical block c at level l    */
/* (l = 0..3) covers pooled rows [c*bk/2^l, (c+1)*bk/2^l) of region l,      */
/* i.e. eighths (bk/8 rows each) of augmented block                         */
/* region_block[l] + c*bk/2^l / bk. Per row: every augmented block with at  */
/* least one selected eighth, in ascending block order, with the bit mask   */
/* of its selected eighths (bit i = rows i*bk/8 .. (i+1)*bk/8 - 1).         */
int64_t oracle_compact_pyramid(int64_t B, int64_t H, int64_t nQ, int64_t nK, int64_t N,
                               int64_t bk, int64_t n_levels, const uint8_t* mask,
                               int64_t mask_head_stride, int32_t* row_ptr, int32_t* kv_idx,
                               uint8_t* kv_eighths) {
  int64_t rb[5], rr[5];
  if (n_levels < 1 || n_levels > 4) return -1;
  oracle_pyramid_regions(N, bk, n_levels, rb, rr);
  int64_t nA = rb[n_levels];
  uint8_t* qm = (uint8_t*)calloc((size_t)(nA > 0 ? nA : 1), 1);
  if (!qm) return -1;
  int64_t nnz = 0;
  int bad = 0;
  for (int64_t bh = 0; bh < B * H; ++bh)
    for (int64_t a = 0; a < nQ; ++a) {
      int64_t r = bh * nQ + a;
      if (row_ptr) row_ptr[r] = (int32_t)nnz;
      memset(qm, 0, (size_t)nA);
      for (int64_t c = 0; c < nK; ++c) {
        int v = mask[bh * mask_head_stride + a * nK + c];
        if (!v) continue;
        if (v > n_levels) {                          /* not a level of this pyramid */
          bad = 1;
          continue;
        }
        int64_t l = v - 1, per = bk >> l;          /* pooled rows of the block */
        int64_t row0 = c * per;                      /* first pooled row in region */
        for (int64_t rr0 = row0; rr0 < row0 + per; rr0 += bk / 8)
          qm[rb[l] + rr0 / bk] |= (uint8_t)(1u << ((rr0 % bk) / (bk / 8)));
      }
      for (int64_t ab = 0; ab < nA; ++ab)
        if (qm[ab]) {
          if (kv_idx) kv_idx[nnz] = (int32_t)ab;
          if (kv_eighths) kv_eighths[nnz] = qm[ab];
          ++nnz;
        }
    }
  if (row_ptr) row_ptr[B * H * nQ] = (int32_t)nnz;
  free(qm);
  return bad ? -1 : nnz;
}

/* ------------------------------------------------------------------------ */
/* Masked softmax attention (the plain definition the kernels reach by an    */
/* exact re-association; bidirectional, no causal mask). For query i of row  */
/* block a of head (b, h), J_i is the union of the column blocks c with      */
/* mask(b, h, a, c) = 1, and                                                 */
/*   s_ij = scale * sum_x q_ix k_jx,  m_i = max_{j in J_i} s_ij,              */
/*   l_i = sum_{j in J_i} exp(s_ij - m_i),                                   */
/*   o_i = sum_{j in J_i} exp(s_ij - m_i) v_j / l_i,  lse_i = m_i + log l_i;  */
/* empty J_i gives o_i = 0, lse_i = -inf.                                    */
/*                                                                           */
/* Tile gaps ([Lite] section 五: a tile whose local maximum lies far below   */
/* the accumulated maximum contributes exponentially little; section 六:     */
/* per-warp decisions combined across warps): visiting the kept column      */
/* blocks of row block a in ascending order (order 0) or in the radial-     */
/* centric order of oracle_order_lists (order 1), with m_run(r) = -inf at   */
/* start,                                                                    */
/*   m_loc(r) = max_{j in C_c} s_rj,                                          */
/*   gap(a, c) = max over valid rows r of (m_loc(r) - m_run(r)),              */
/*   m_run(r) = max(m_run(r), m_loc(r)).                                      */
/* Natural-log units of the scaled scores; +inf for the first visited tile.  */
/*                                                                           */
/* Only the requested rows are computed: rows[t] = (b*H + h)*nQ + a.         */
/* Outputs: o_out [n_rows][bq][D], lse_out [n_rows][bq] (padding rows of a   */
/* ragged last block are NaN), gap_out [n_rows][nK] (NaN where not kept),    */
/* each optional.                                                            */
/* ------------------------------------------------------------------------ */
int oracle_attention(int64_t B, int64_t H, int64_t N, int64_t D, int64_t bq,
                     int64_t bk, int dtype,
                     const void* q, int64_t qsb, int64_t qsn, int64_t qsh,
                     const void* k, int64_t ksb, int64_t ksn, int64_t ksh,
                     const void* v, int64_t vsb, int64_t vsn, int64_t vsh,
                     double scale, const uint8_t* mask, int64_t mask_head_stride,
                     int64_t n_rows, const int64_t* rows,
                     double* o_out, double* lse_out, double* gap_out, int order) {
  int64_t nQ = (N + bq - 1) / bq, nK = (N + bk - 1) / bk;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < n_rows; ++t) {
    int64_t row = rows[t];
    int64_t bh = row / nQ, a = row % nQ, b = bh / H, h = bh % H;
    int64_t i0 = a * bq, i1 = (a + 1) * bq < N ? (a + 1) * bq : N;
    const uint8_t* m = mask + bh * mask_head_stride + a * nK;
    int64_t nJ = 0;
    for (int64_t c = 0; c < nK; ++c)
      if (m[c]) nJ += ((c + 1) * bk < N ? (c + 1) * bk : N) - c * bk;
    double* s = (double*)malloc(sizeof(double) * (nJ > 0 ? nJ : 1));
    double* qi = (double*)malloc(sizeof(double) * D);
    double* acc = (double*)malloc(sizeof(double) * D);
    double* mrun = (double*)malloc(sizeof(double) * bq);
    double* mblk = (double*)malloc(sizeof(double) * nK);
    int32_t* visit = (int32_t*)malloc(sizeof(int32_t) * (nK > 0 ? nK : 1));
    if (!s || !qi || !acc || !mrun || !mblk || !visit) {
#pragma omp atomic write
      bad = 1;
      free(s); free(qi); free(acc); free(mrun); free(mblk); free(visit);
      continue;
    }
    /* the kept blocks of this row in visiting order */
    int64_t n_visit = 0;
    for (int64_t c = 0; c < nK; ++c)
      if (m[c]) visit[n_visit++] = (int32_t)c;
    if (order == 1) radial_sort(visit, n_visit, block_mid2(a, bq, N), bk, N);
    for (int64_t r = 0; r < bq; ++r) mrun[r] = -INFINITY;
    if (gap_out)
      for (int64_t c = 0; c < nK; ++c) gap_out[t * nK + c] = NAN;
    for (int64_t r = 0; r < bq; ++r) {
      if (o_out) for (int64_t x = 0; x < D; ++x) o_out[(t * bq + r) * D + x] = NAN;
      if (lse_out) lse_out[t * bq + r] = NAN;
    }
    for (int64_t i = i0; i < i1; ++i) {
      int64_t r = i - i0;
      for (int64_t x = 0; x < D; ++x) qi[x] = widen(q, dtype, b * qsb + i * qsn + h * qsh + x);
      /* scores over J_i, in ascending j */
      int64_t n = 0;
      for (int64_t c = 0; c < nK; ++c) {
        if (!m[c]) continue;
        int64_t j0 = c * bk, j1 = (c + 1) * bk < N ? (c + 1) * bk : N;
        double mloc = -INFINITY;
        for (int64_t j = j0; j < j1; ++j) {
          double dot = 0.0;
          for (int64_t x = 0; x < D; ++x)
            dot = dot + qi[x] * widen(k, dtype, b * ksb + j * ksn + h * ksh + x);
          s[n++] = scale * dot;
          if (s[n - 1] > mloc) mloc = s[n - 1];
        }
        mblk[c] = mloc;
      }
      /* gaps: the kept blocks in visiting order against the running max */
      for (int64_t u = 0; u < n_visit; ++u) {
        int64_t c = visit[u];
        if (gap_out) {
          double g = mblk[c] - mrun[r]; /* +inf on the first visited tile */
          double* gp = &gap_out[t * nK + c];
          if (isnan(*gp) || g > *gp) *gp = g;
        }
        if (mblk[c] > mrun[r]) mrun[r] = mblk[c];
      }
      if (nJ == 0) {
        if (o_out) for (int64_t x = 0; x < D; ++x) o_out[(t * bq + r) * D + x] = 0.0;
        if (lse_out) lse_out[t * bq + r] = -INFINITY;
        continue;
      }
      double mi = -INFINITY;
      for (int64_t u = 0; u < nJ; ++u) if (s[u] > mi) mi = s[u];
      double li = 0.0;
      for (int64_t u = 0; u < nJ; ++u) li = li + exp(s[u] - mi);
      for (int64_t x = 0; x < D; ++x) acc[x] = 0.0;
      n = 0;
      for (int64_t c = 0; c < nK; ++c) {
        if (!m[c]) continue;
        int64_t j0 = c * bk, j1 = (c + 1) * bk < N ? (c + 1) * bk : N;
        for (int64_t j = j0; j < j1; ++j) {
          double p = exp(s[n++] - mi);
          for (int64_t x = 0; x < D; ++x)
            acc[x] = acc[x] + p * widen(v, dtype, b * vsb + j * vsn + h * vsh + x);
        }
      }
      if (o_out) for (int64_t x = 0; x < D; ++x) o_out[(t * bq + r) * D + x] = acc[x] / li;
      if (lse_out) lse_out[t * bq + r] = mi + log(li);
    }
    free(s); free(qi); free(acc); free(mrun); free(mblk); free(visit);
  }
  return bad ? -1 : 0;
}
