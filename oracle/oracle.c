/*
 * oracle.c -- plain, slow, double-precision reference for the teacher-forced
 * logit comparison.  TEST INFRASTRUCTURE ONLY: the parity tests, the smoke
 * check and the CPU-baseline leg of the benchmark are its only users.  It
 * shares no code, header, table or constant with the GPU library.
 *
 * Every quantity is computed from its plain definition, row by row, with
 * sequential sums in ascending index order and a full sort for the top-k.
 * OpenMP only splits independent rows between threads; results do not depend
 * on the thread count.
 *
 * Pages cited (by title and section):
 *   [logits]  "在 agent 时代如何快速验证 kernel 对精度的影响" (susun-blog,
 *             verify-kernel-precision-with-logits)
 *   [bitexact] "Kestrel_VLLM - 18 · 投机解码位级对拍收口" (wsisp.com helps/117433)
 *   [dcu]     "海光 DCU 实测：BF16 逐位一致为什么仍可能出现文本漂移" (forum.sourcefind.cn)
 *
 * Readings taken where the pages leave a step open (each one is restated in
 * the design notes of the repository):
 *   - KL is KL(baseline || candidate) in nats, softmax at temperature 1 over
 *     the full vocabulary.
 *   - The top-k set is the baseline's k largest logits, ties broken by the
 *     lower index; the "other" bucket is the complement, summed on each side.
 *   - The candidate's top-1 is the lowest index among its maximal logits.
 *   - margin = x[top1] - x[top2] of the baseline, one double subtraction.
 *   - A row holding NaN or +inf on either side is flagged NONFINITE; a row
 *     whose baseline or candidate is entirely -inf is flagged EMPTY.  Flagged
 *     rows report NaN / -1 / 0 in every other field.
 *   - ULP distance uses the monotone integer ordering o(u) = u | signbit for
 *     patterns with a clear sign bit and o(u) = ~u otherwise, so +0 and -0
 *     are one unit apart and "bits differ" equals "nonzero ULP distance".
 *   - Bitwise error norms are taken over positions where both values are
 *     finite; non-finite elements are counted per side.
 *   - Margin bins are half-open [e_{j-1}, e_j) with e_{-1} = 0; a flip at
 *     margin strictly above the big-margin threshold is a big-margin flip.
 *   - The target log-probability of a flagged row, or of a target outside
 *     [0, v), is NaN.
 *   - A stored baseline record keeps the k largest logits with their indices
 *     and the log of the remaining mass; its status is the baseline's alone.
 *     Comparing a candidate against it flags NONFINITE when either the record
 *     or the candidate is NONFINITE, else EMPTY when either is EMPTY.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* dtype codes of the oracle's own interface */
#define ORC_F32 0
#define ORC_BF16 1

#define ORC_ROW_NONFINITE 1
#define ORC_ROW_EMPTY 2

/* ------------------------------------------------------------------ decoding */

static uint32_t pattern32(const void *row, int dtype, int64_t i) {
  if (dtype == ORC_BF16) return (uint32_t)((const uint16_t *)row)[i] << 16;
  return ((const uint32_t *)row)[i];
}

/* exact widening of an element to double */
static double value(const void *row, int dtype, int64_t i) {
  uint32_t u = pattern32(row, dtype, i);
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* -------------------------------------------------------- softmax statistics */

/* log of the softmax normaliser: m + log(sum_i exp(x_i - m)), summed in index
 * order ([logits] 怎么比两个分布: p_i is the softmax of the logits). */
static double log_normaliser(const double *x, int64_t v) {
  double m = -INFINITY;
  for (int64_t i = 0; i < v; i++)
    if (x[i] > m) m = x[i];
  if (m == -INFINITY) return -INFINITY;
  double s = 0.0;
  for (int64_t i = 0; i < v; i++) s += exp(x[i] - m);
  return m + log(s);
}

/* ------------------------------------------------------------ top-k ordering */

typedef struct {
  double x;
  int64_t i;
} keyed;

/* value descending, index ascending */
static int by_value_desc(const void *pa, const void *pb) {
  const keyed *a = (const keyed *)pa, *b = (const keyed *)pb;
  if (a->x > b->x) return -1;
  if (a->x < b->x) return 1;
  return (a->i < b->i) ? -1 : (a->i > b->i);
}

/* ------------------------------------------------------------ one row compare */

typedef struct {
  double kl_topk, kl_full, margin, lse_base, lse_cand;
  int32_t top1_base, top2_base, top1_cand;
  uint8_t flip, status;
} orc_row;

static void flag_row(orc_row *o, uint8_t status, int32_t *topk_idx, int k) {
  o->kl_topk = o->kl_full = o->margin = o->lse_base = o->lse_cand = NAN;
  o->top1_base = o->top2_base = o->top1_cand = -1;
  o->flip = 0;
  o->status = status;
  for (int j = 0; j < k; j++) topk_idx[j] = -1;
}

/* the finite check of the ladder in [dcu] §1 / §7: a NaN or +inf on either
 * side flags the row NONFINITE, a side that is entirely -inf flags it EMPTY */
static uint8_t row_status(const double *x, const double *y, int64_t v) {
  int bad = 0, x_any = 0, y_any = 0;
  for (int64_t i = 0; i < v; i++) {
    if (isnan(x[i]) || isnan(y[i]) || x[i] == INFINITY || y[i] == INFINITY) bad = 1;
    if (x[i] > -INFINITY) x_any = 1;
    if (y[i] > -INFINITY) y_any = 1;
  }
  if (bad) return ORC_ROW_NONFINITE;
  if (!x_any || !y_any) return ORC_ROW_EMPTY;
  return 0;
}

static void compare_row(const double *x, const double *y, int64_t v, int k, keyed *order,
                        orc_row *o, int32_t *topk_idx) {
  const uint8_t st = row_status(x, y, v);
  if (st) {
    flag_row(o, st, topk_idx, k);
    return;
  }
  const int64_t keff = (int64_t)k < v ? (int64_t)k : v;

  const double lse_a = log_normaliser(x, v);
  const double lse_b = log_normaliser(y, v);
  o->lse_base = lse_a;
  o->lse_cand = lse_b;

  /* full KL(P||Q) = sum_i p_i (ln p_i - ln q_i) ([logits] 怎么比两个分布, KL equation).
   * Tokens with p_i = 0 add nothing; p_i > 0 with q_i = 0 makes it infinite. */
  double kl = 0.0;
  int inf_full = 0;
  for (int64_t i = 0; i < v; i++) {
    if (x[i] == -INFINITY) continue;
    if (y[i] == -INFINITY) {
      inf_full = 1;
      continue;
    }
    const double lp = x[i] - lse_a, lq = y[i] - lse_b;
    kl += exp(lp) * (lp - lq);
  }
  o->kl_full = inf_full ? INFINITY : kl;

  /* baseline top-k by a full sort ([logits] 怎么比两个分布, top-20 + "other") */
  for (int64_t i = 0; i < v; i++) {
    order[i].x = x[i];
    order[i].i = i;
  }
  qsort(order, (size_t)v, sizeof(keyed), by_value_desc);
  for (int j = 0; j < k; j++) topk_idx[j] = j < keff ? (int32_t)order[j].i : -1;

  /* top-k + other KL: head tokens term by term, the rest merged into one bucket
   * on each side. */
  double klk = 0.0;
  int inf_k = 0;
  for (int64_t j = 0; j < keff; j++) {
    const int64_t i = order[j].i;
    if (x[i] == -INFINITY) continue;
    if (y[i] == -INFINITY) {
      inf_k = 1;
      continue;
    }
    const double lp = x[i] - lse_a, lq = y[i] - lse_b;
    klk += exp(lp) * (lp - lq);
  }
  /* bucket masses in log form: log p_o = log sum_{i not in S} exp(x_i - lse_a) */
  double mo_x = -INFINITY, mo_y = -INFINITY;
  for (int64_t j = keff; j < v; j++) {
    const int64_t i = order[j].i;
    if (x[i] > mo_x) mo_x = x[i];
    if (y[i] > mo_y) mo_y = y[i];
  }
  if (mo_x > -INFINITY) {
    if (mo_y == -INFINITY) {
      inf_k = 1; /* baseline mass in the bucket, none on the candidate side */
    } else {
      double sx = 0.0, sy = 0.0;
      for (int64_t j = keff; j < v; j++) {
        const int64_t i = order[j].i;
        sx += exp(x[i] - mo_x);
        sy += exp(y[i] - mo_y);
      }
      const double lpo = mo_x - lse_a + log(sx), lqo = mo_y - lse_b + log(sy);
      klk += exp(lpo) * (lpo - lqo);
    }
  }
  o->kl_topk = inf_k ? INFINITY : klk;

  /* margin: baseline top-1 logit minus top-2 logit ([logits] 怎么比两个分布, margin) */
  o->top1_base = (int32_t)order[0].i;
  o->top2_base = (int32_t)order[1].i;
  o->margin = order[0].x - order[1].x;

  /* candidate top-1 (lowest index among the maxima) and the flip
   * ([logits] 怎么比两个分布, top-1 翻转) */
  int64_t best = 0;
  for (int64_t i = 1; i < v; i++)
    if (y[i] > y[best]) best = i;
  o->top1_cand = (int32_t)best;
  o->flip = (uint8_t)(best != order[0].i);
  o->status = 0;
}

/*
 * Compare n rows.  base/cand: row-major with leading dimensions in elements.
 * Any output pointer may be NULL.  topk_idx is [n, k].  Returns 0, or -1 on
 * a bad argument or allocation failure.
 */
int orc_compare(const void *base, int tb, int64_t ld_base, const void *cand, int tc,
                int64_t ld_cand, int64_t n, int64_t v, int k, double *kl_topk, double *kl_full,
                double *margin, double *lse_base, double *lse_cand, int32_t *top1_base,
                int32_t *top2_base, int32_t *top1_cand, uint8_t *flip, int32_t *topk_idx,
                uint8_t *status, int nthreads) {
  if (!base || !cand || n < 0 || v < 2 || k < 1 || ld_base < v || ld_cand < v) return -1;
  if ((tb != ORC_F32 && tb != ORC_BF16) || (tc != ORC_F32 && tc != ORC_BF16)) return -1;
  const size_t eb = tb == ORC_BF16 ? 2 : 4, ec = tc == ORC_BF16 ? 2 : 4;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double *x = (double *)malloc((size_t)v * sizeof(double));
    double *y = (double *)malloc((size_t)v * sizeof(double));
    keyed *order = (keyed *)malloc((size_t)v * sizeof(keyed));
    int32_t *idx = (int32_t *)malloc((size_t)k * sizeof(int32_t));
    if (!x || !y || !order || !idx) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; r++) {
      if (!x || !y || !order || !idx) continue;
      const void *br = (const char *)base + (size_t)r * (size_t)ld_base * eb;
      const void *cr = (const char *)cand + (size_t)r * (size_t)ld_cand * ec;
      for (int64_t i = 0; i < v; i++) {
        x[i] = value(br, tb, i);
        y[i] = value(cr, tc, i);
      }
      orc_row o;
      compare_row(x, y, v, k, order, &o, idx);
      if (kl_topk) kl_topk[r] = o.kl_topk;
      if (kl_full) kl_full[r] = o.kl_full;
      if (margin) margin[r] = o.margin;
      if (lse_base) lse_base[r] = o.lse_base;
      if (lse_cand) lse_cand[r] = o.lse_cand;
      if (top1_base) top1_base[r] = o.top1_base;
      if (top2_base) top2_base[r] = o.top2_base;
      if (top1_cand) top1_cand[r] = o.top1_cand;
      if (flip) flip[r] = o.flip;
      if (status) status[r] = o.status;
      if (topk_idx) memcpy(topk_idx + (size_t)r * (size_t)k, idx, (size_t)k * sizeof(int32_t));
    }
    free(x);
    free(y);
    free(order);
    free(idx);
  }
  return failed ? -1 : 0;
}

/* ------------------------------------------------------ target log-probability */

/*
 * ln p(target) and ln q(target) of each row: the teacher-forced next token's
 * log-probability under the baseline and the candidate softmax, the only
 * number perplexity keeps of a distribution ([logits] perplexity（困惑度）看不出
 * 这一级的差别).  NaN for a flagged row or a target outside [0, v).
 */
int orc_target_logprob(const void *base, int tb, int64_t ld_base, const void *cand, int tc,
                       int64_t ld_cand, int64_t n, int64_t v, const int32_t *target,
                       double *logp_base, double *logp_cand, int nthreads) {
  if (!base || !cand || !target || !logp_base || !logp_cand || n < 0 || v < 2 ||
      ld_base < v || ld_cand < v)
    return -1;
  if ((tb != ORC_F32 && tb != ORC_BF16) || (tc != ORC_F32 && tc != ORC_BF16)) return -1;
  const size_t eb = tb == ORC_BF16 ? 2 : 4, ec = tc == ORC_BF16 ? 2 : 4;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double *x = (double *)malloc((size_t)v * sizeof(double));
    double *y = (double *)malloc((size_t)v * sizeof(double));
    if (!x || !y) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; r++) {
      if (!x || !y) continue;
      const void *br = (const char *)base + (size_t)r * (size_t)ld_base * eb;
      const void *cr = (const char *)cand + (size_t)r * (size_t)ld_cand * ec;
      for (int64_t i = 0; i < v; i++) {
        x[i] = value(br, tb, i);
        y[i] = value(cr, tc, i);
      }
      const int32_t t = target[r];
      if (row_status(x, y, v) != 0 || t < 0 || (int64_t)t >= v) {
        logp_base[r] = NAN;
        logp_cand[r] = NAN;
        continue;
      }
      logp_base[r] = x[t] - log_normaliser(x, v);
      logp_cand[r] = y[t] - log_normaliser(y, v);
    }
    free(x);
    free(y);
  }
  return failed ? -1 : 0;
}

/* ------------------------------------------------------ compact ground-truth record */

/*
 * The ground truth is run once and its distributions are stored; every later
 * candidate is compared against that store, never against a previous candidate
 * ([logits] 先要有一个 ground truth).  What the top-k comparison needs of a
 * baseline row is its k largest logits with their indices and the mass of the
 * rest, so that is what a record keeps:
 *   idx[j], val[j]  the baseline's k largest logits (value descending, index
 *                   ascending; -1 and -inf past min(k, v))
 *   lse_rest        ln sum_{i not in the top k} exp(x_i); -inf when nothing is left
 *   status          NONFINITE (a NaN or +inf) or EMPTY (all -inf) of the baseline
 *                   alone; a flagged row holds -1 / NaN everywhere
 *   logp_target     optional: ln p(target) = x[target] - ln sum_i exp(x_i)
 */
int orc_record(const void *base, int tb, int64_t ld_base, int64_t n, int64_t v, int k,
               const int32_t *target, int32_t *idx, float *val, double *lse_rest,
               uint8_t *status, double *logp_target, int nthreads) {
  if (!base || !idx || !val || !lse_rest || !status || n < 0 || v < 2 || k < 2 || ld_base < v)
    return -1;
  if (tb != ORC_F32 && tb != ORC_BF16) return -1;
  if (logp_target && !target) return -1;
  const size_t eb = tb == ORC_BF16 ? 2 : 4;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double *x = (double *)malloc((size_t)v * sizeof(double));
    keyed *order = (keyed *)malloc((size_t)v * sizeof(keyed));
    if (!x || !order) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; r++) {
      if (!x || !order) continue;
      const void *br = (const char *)base + (size_t)r * (size_t)ld_base * eb;
      for (int64_t i = 0; i < v; i++) x[i] = value(br, tb, i);
      int32_t *ri = idx + (size_t)r * (size_t)k;
      float *rv = val + (size_t)r * (size_t)k;
      const uint8_t st = row_status(x, x, v);
      status[r] = st;
      if (st) {
        for (int j = 0; j < k; j++) {
          ri[j] = -1;
          rv[j] = NAN;
        }
        lse_rest[r] = NAN;
        if (logp_target) logp_target[r] = NAN;
        continue;
      }
      for (int64_t i = 0; i < v; i++) {
        order[i].x = x[i];
        order[i].i = i;
      }
      qsort(order, (size_t)v, sizeof(keyed), by_value_desc);
      const int64_t keff = (int64_t)k < v ? (int64_t)k : v;
      for (int j = 0; j < k; j++) {
        ri[j] = j < keff ? (int32_t)order[j].i : -1;
        rv[j] = j < keff ? (float)order[j].x : -INFINITY;
      }
      double m = -INFINITY;
      for (int64_t j = keff; j < v; j++)
        if (order[j].x > m) m = order[j].x;
      if (m == -INFINITY) {
        lse_rest[r] = -INFINITY;
      } else {
        double s = 0.0;
        for (int64_t j = keff; j < v; j++) s += exp(order[j].x - m);
        lse_rest[r] = m + log(s);
      }
      if (logp_target) {
        const int32_t t = target[r];
        logp_target[r] = (t < 0 || (int64_t)t >= v) ? NAN : x[t] - log_normaliser(x, v);
      }
    }
    free(x);
    free(order);
  }
  return failed ? -1 : 0;
}

/* ln(exp(a) + exp(b)) */
static double log_add(double a, double b) {
  if (a == -INFINITY) return b;
  if (b == -INFINITY) return a;
  const double m = a > b ? a : b;
  return m + log(exp(a - m) + exp(b - m));
}

/*
 * Compare candidate rows against a record of k_rec entries per row, using its
 * first k (k <= k_rec): the same top-k + "other" KL, margin, flip, top-1 and
 * normalisers as the full compare ([logits] 怎么比两个分布), from the record and
 * the candidate row alone.  The baseline distribution over the head and the
 * bucket is rebuilt from the record: ln p_j = val_j - L, ln p_o = R - L with
 * R = ln(sum_{k <= j < k_rec} exp(val_j) + exp(lse_rest)) and L = ln(sum_{j<k}
 * exp(val_j) + exp(R)).  The candidate's bucket is summed directly over the
 * columns outside the head.  The full KL needs the whole baseline row and is
 * not produced.  Status: NONFINITE if either the record or the candidate is
 * NONFINITE, else EMPTY if either is EMPTY.
 */
int orc_compare_record(const int32_t *idx, const float *val, const double *lse_rest,
                       const uint8_t *rec_status, const double *rec_logp, int k_rec,
                       const void *cand, int tc, int64_t ld_cand, int64_t n, int64_t v, int k,
                       const int32_t *target, double *kl_topk, double *margin, double *lse_base,
                       double *lse_cand, int32_t *top1_base, int32_t *top2_base,
                       int32_t *top1_cand, uint8_t *flip, int32_t *topk_idx, uint8_t *status,
                       double *logp_base, double *logp_cand, int nthreads) {
  if (!idx || !val || !lse_rest || !rec_status || !cand || n < 0 || v < 2 || k < 1 ||
      k_rec < 2 || k > k_rec || ld_cand < v)
    return -1;
  if (tc != ORC_F32 && tc != ORC_BF16) return -1;
  if ((logp_base && !rec_logp) || ((logp_base || logp_cand) && !target)) return -1;
  const size_t ec = tc == ORC_BF16 ? 2 : 4;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel
  {
    double *y = (double *)malloc((size_t)v * sizeof(double));
    unsigned char *in_head = (unsigned char *)malloc((size_t)v);
    if (!y || !in_head) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n; r++) {
      if (!y || !in_head) continue;
      const void *cr = (const char *)cand + (size_t)r * (size_t)ld_cand * ec;
      for (int64_t i = 0; i < v; i++) y[i] = value(cr, tc, i);
      const int32_t *ri = idx + (size_t)r * (size_t)k_rec;
      const float *rv = val + (size_t)r * (size_t)k_rec;
      const uint8_t sc = row_status(y, y, v);
      const uint8_t sr = rec_status[r];
      const uint8_t st = (sr == ORC_ROW_NONFINITE || sc == ORC_ROW_NONFINITE) ? ORC_ROW_NONFINITE
                         : (sr || sc)                                          ? ORC_ROW_EMPTY
                                                                               : 0;
      if (status) status[r] = st;
      if (topk_idx)
        for (int j = 0; j < k; j++) topk_idx[(size_t)r * k + j] = st ? -1 : ri[j];
      if (st) {
        if (kl_topk) kl_topk[r] = NAN;
        if (margin) margin[r] = NAN;
        if (lse_base) lse_base[r] = NAN;
        if (lse_cand) lse_cand[r] = NAN;
        if (top1_base) top1_base[r] = -1;
        if (top2_base) top2_base[r] = -1;
        if (top1_cand) top1_cand[r] = -1;
        if (flip) flip[r] = 0;
        if (logp_base) logp_base[r] = NAN;
        if (logp_cand) logp_cand[r] = NAN;
        continue;
      }
      /* baseline side from the record */
      double R = lse_rest[r];
      for (int j = k; j < k_rec; j++)
        if (ri[j] >= 0) R = log_add(R, (double)rv[j]);
      double L = R;
      for (int j = 0; j < k; j++)
        if (ri[j] >= 0) L = log_add(L, (double)rv[j]);
      /* candidate side: full normaliser, and the bucket over columns outside the head */
      const double lse_y = log_normaliser(y, v);
      memset(in_head, 0, (size_t)v);
      for (int j = 0; j < k; j++)
        if (ri[j] >= 0) in_head[ri[j]] = 1;
      double mo = -INFINITY;
      for (int64_t i = 0; i < v; i++)
        if (!in_head[i] && y[i] > mo) mo = y[i];
      double Ry = -INFINITY;
      if (mo > -INFINITY) {
        double s = 0.0;
        for (int64_t i = 0; i < v; i++)
          if (!in_head[i]) s += exp(y[i] - mo);
        Ry = mo + log(s);
      }
      /* top-k + other KL, with the infinite cases of the full compare */
      double klk = 0.0;
      int inf_k = 0;
      for (int j = 0; j < k; j++) {
        if (ri[j] < 0 || rv[j] == -INFINITY) continue;
        const double yj = y[ri[j]];
        if (yj == -INFINITY) {
          inf_k = 1;
          continue;
        }
        const double lp = (double)rv[j] - L, lq = yj - lse_y;
        klk += exp(lp) * (lp - lq);
      }
      if (R > -INFINITY) {
        if (Ry == -INFINITY) {
          inf_k = 1;
        } else {
          const double lpo = R - L, lqo = Ry - lse_y;
          klk += exp(lpo) * (lpo - lqo);
        }
      }
      int64_t best = 0;
      for (int64_t i = 1; i < v; i++)
        if (y[i] > y[best]) best = i;
      if (kl_topk) kl_topk[r] = inf_k ? INFINITY : klk;
      if (margin) margin[r] = (double)rv[0] - (double)rv[1];
      if (lse_base) lse_base[r] = L;
      if (lse_cand) lse_cand[r] = lse_y;
      if (top1_base) top1_base[r] = ri[0];
      if (top2_base) top2_base[r] = ri[1];
      if (top1_cand) top1_cand[r] = (int32_t)best;
      if (flip) flip[r] = (uint8_t)(best != ri[0]);
      if (logp_base || logp_cand) {
        const int32_t t = target[r];
        const int ok = t >= 0 && (int64_t)t < v;
        if (logp_base) logp_base[r] = ok ? rec_logp[r] : NAN;
        if (logp_cand) logp_cand[r] = ok ? y[t] - lse_y : NAN;
      }
    }
    free(y);
    free(in_head);
  }
  return failed ? -1 : 0;
}

/* ------------------------------------------------------ precision perturbations */

/*
 * The precision-knee experiments of [logits] (实验 section): keep only m
 * fraction bits of an fp32 value with the exponent range unchanged, or round
 * to fp8 e4m3 directly or after scaling by 448 (注意力权重 paragraph; the
 * round_p variants).  Round to nearest, ties to even, written from the value:
 * the quantum is 2^(E - m) with E = max(floor(log2 |x|), emin), the multiple
 * of the quantum nearest to x is taken in double (exact: the quantum is a
 * power of two), and the result converted back.  NaN stays NaN.
 */
#define ORC_PERTURB_MANTISSA 0
#define ORC_PERTURB_E4M3 1
#define ORC_PERTURB_E4M3_SCALED 2

static double round_to_quantum(double x, int m, int emin) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  frexp(x, &e); /* x = f * 2^e, 0.5 <= |f| < 1, so floor(log2 |x|) = e - 1 */
  int E = e - 1;
  if (E < emin) E = emin;
  const double q = ldexp(1.0, E - m);
  return rint(x / q) * q; /* rint: ties to even in the default rounding mode */
}

/* fp32 with m fraction bits: emin -126 (subnormals keep the fp32 quantum grid) */
static float keep_mantissa(float x, int m) {
  if (isnan(x)) return x;
  return (float)round_to_quantum((double)x, m, -126); /* beyond FLT_MAX: inf */
}

/* OCP e4m3 (fn): 3 fraction bits, emin -6 (smallest subnormal 2^-9), largest
 * finite 448, no infinity; out-of-range values saturate to +-448 */
static float to_e4m3(float x) {
  if (isnan(x)) return x;
  double r = round_to_quantum((double)x, 3, -6);
  if (r > 448.0) r = 448.0;
  if (r < -448.0) r = -448.0;
  return (float)r;
}

static float perturb_value(float x, int mode, int param) {
  if (mode == ORC_PERTURB_MANTISSA) return keep_mantissa(x, param);
  if (mode == ORC_PERTURB_E4M3) return to_e4m3(x);
  /* scaled: the product and the quotient are fp32 operations, as in the listing
   * of the page's round_p ("fp8, scaled by 448") */
  const float t = x * 448.0f;
  return to_e4m3(t) / 448.0f;
}

/*
 * dst[r, c] = perturb(src[r, c]) for r < rows, c < cols.  src is fp32 or bf16
 * (widened exactly); dst is fp32, or bf16 when every result is representable
 * there (mantissa modes with m <= 7, and plain e4m3).  Returns 0 or -1.
 */
int orc_perturb(const void *src, int ts, int64_t ld_src, void *dst, int td, int64_t ld_dst,
                int64_t rows, int64_t cols, int mode, int param) {
  if (!src || !dst || rows < 0 || cols < 0 || ld_src < cols || ld_dst < cols) return -1;
  if ((ts != ORC_F32 && ts != ORC_BF16) || (td != ORC_F32 && td != ORC_BF16)) return -1;
  if (mode < ORC_PERTURB_MANTISSA || mode > ORC_PERTURB_E4M3_SCALED) return -1;
  if (mode == ORC_PERTURB_MANTISSA && (param < 0 || param > 23)) return -1;
  if (td == ORC_BF16 && !((mode == ORC_PERTURB_MANTISSA && param <= 7) || mode == ORC_PERTURB_E4M3))
    return -1;
  const size_t es = ts == ORC_BF16 ? 2 : 4, ed = td == ORC_BF16 ? 2 : 4;
  for (int64_t r = 0; r < rows; r++) {
    const void *sr = (const char *)src + (size_t)r * (size_t)ld_src * es;
    char *dr = (char *)dst + (size_t)r * (size_t)ld_dst * ed;
    for (int64_t c = 0; c < cols; c++) {
      const float y = perturb_value((float)value(sr, ts, c), mode, param);
      if (td == ORC_F32) {
        memcpy(dr + 4 * c, &y, 4);
      } else {
        uint32_t u;
        memcpy(&u, &y, 4);
        /* exact: y has at most 7 fraction bits; a NaN keeps its quiet bit */
        const uint16_t h = (uint16_t)((u >> 16) | (isnan(y) ? 0x0040u : 0u));
        memcpy(dr + 2 * c, &h, 2);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------ bitwise / ULP */

typedef struct {
  int64_t ndiff, first_diff, nonfinite_a, nonfinite_b;
  uint32_t max_ulp, pad_;
  double max_abs, sum_abs, sum_sq_diff, sum_sq_base, mean_abs, rel_l2;
} orc_bitdiff_row;

/* monotone integer image of a bit pattern of the given width (16 or 32) */
static uint32_t ordered(uint32_t u, int width) {
  const uint32_t sign = width == 16 ? 0x8000u : 0x80000000u;
  const uint32_t all = width == 16 ? 0xffffu : 0xffffffffu;
  return (u & sign) ? (~u & all) : (u | sign);
}

/*
 * Per-row bitwise statistics between a and b ([bitexact] 二: full-logit
 * compare as integers, count of differing elements and first differing
 * position; [dcu] §1 and §7: finite check, max abs, mean abs, relative L2).
 * Same dtype: patterns compared at that width.  Mixed dtypes: both sides
 * widened to fp32 patterns (bf16 -> bits << 16), compared at width 32.
 */
int orc_bitdiff(const void *a, int ta, int64_t lda, const void *b, int tb, int64_t ldb,
                int64_t rows, int64_t cols, orc_bitdiff_row *out, int nthreads) {
  if (!a || !b || !out || rows < 0 || cols < 1 || lda < cols || ldb < cols) return -1;
  if ((ta != ORC_F32 && ta != ORC_BF16) || (tb != ORC_F32 && tb != ORC_BF16)) return -1;
  const int width = (ta == ORC_BF16 && tb == ORC_BF16) ? 16 : 32;
  const size_t ea = ta == ORC_BF16 ? 2 : 4, eb = tb == ORC_BF16 ? 2 : 4;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; r++) {
    const void *ar = (const char *)a + (size_t)r * (size_t)lda * ea;
    const void *br = (const char *)b + (size_t)r * (size_t)ldb * eb;
    orc_bitdiff_row o;
    memset(&o, 0, sizeof o);
    o.first_diff = -1;
    for (int64_t i = 0; i < cols; i++) {
      uint32_t ua = pattern32(ar, ta, i), ub = pattern32(br, tb, i);
      if (width == 16) {
        ua >>= 16;
        ub >>= 16;
      }
      if (ua != ub) {
        o.ndiff++;
        if (o.first_diff < 0) o.first_diff = i;
      }
      const int64_t d = (int64_t)ordered(ua, width) - (int64_t)ordered(ub, width);
      const uint32_t ulp = (uint32_t)(d < 0 ? -d : d);
      if (ulp > o.max_ulp) o.max_ulp = ulp;
      const double x = value(ar, ta, i), y = value(br, tb, i);
      const int fx = isfinite(x), fy = isfinite(y);
      if (!fx) o.nonfinite_a++;
      if (!fy) o.nonfinite_b++;
      if (fx && fy) {
        const double e = x - y;
        if (fabs(e) > o.max_abs) o.max_abs = fabs(e);
        o.sum_abs += fabs(e);
        o.sum_sq_diff += e * e;
        o.sum_sq_base += x * x;
      }
    }
    o.mean_abs = o.sum_abs / (double)cols;
    if (o.sum_sq_base > 0.0)
      o.rel_l2 = sqrt(o.sum_sq_diff / o.sum_sq_base);
    else
      o.rel_l2 = o.sum_sq_diff > 0.0 ? INFINITY : 0.0;
    out[r] = o;
  }
  return 0;
}

/* ------------------------------------------------------------ margin bins */

typedef struct {
  int64_t count, flips, ties, tie_flips;
  double sum_kl_topk, sum_kl_full, max_kl_topk;
} orc_bin;

typedef struct {
  int64_t big_margin_flips, excluded, unbinned;
} orc_group_summary;

/*
 * Flip rates by margin bin ([logits] 三者联合起来验证精度问题: count flips per
 * margin bin and compare each bin with the normal difference; a flip at a
 * margin above 1 calls for a stop).  Rows are taken in ascending order.
 * group may be NULL (one group); rows whose group id is outside
 * [0, n_groups) are skipped; rows with a nonzero status are counted as
 * excluded in their group.  bins is [n_groups, n_edges].
 */
int orc_bin_report(const double *margin, const uint8_t *flip, const double *kl_topk,
                   const double *kl_full, const uint8_t *status, const int32_t *group,
                   int n_groups, int64_t n, const double *edges, int n_edges, double big_margin,
                   orc_bin *bins, orc_group_summary *summary) {
  if (!margin || !flip || !kl_topk || !edges || !bins || !summary) return -1;
  if (n_groups < 1 || n_edges < 1 || n < 0) return -1;
  for (int j = 0; j < n_edges; j++) {
    if (isnan(edges[j]) || edges[j] <= 0.0) return -1;
    if (j > 0 && !(edges[j] > edges[j - 1])) return -1;
  }
  for (int64_t t = 0; t < (int64_t)n_groups * n_edges; t++) {
    memset(&bins[t], 0, sizeof(orc_bin));
    bins[t].max_kl_topk = -INFINITY;
  }
  memset(summary, 0, (size_t)n_groups * sizeof(orc_group_summary));
  for (int64_t r = 0; r < n; r++) {
    const int g = group ? group[r] : 0;
    if (g < 0 || g >= n_groups) continue;
    if (status && status[r] != 0) {
      summary[g].excluded++;
      continue;
    }
    const double m = margin[r];
    if (flip[r] && m > big_margin) summary[g].big_margin_flips++;
    int j = 0;
    while (j < n_edges && !(m < edges[j])) j++;
    if (j == n_edges) {
      summary[g].unbinned++;
      continue;
    }
    orc_bin *bn = &bins[(int64_t)g * n_edges + j];
    bn->count++;
    bn->flips += flip[r] ? 1 : 0;
    if (m == 0.0) {
      bn->ties++;
      bn->tie_flips += flip[r] ? 1 : 0;
    }
    bn->sum_kl_topk += kl_topk[r];
    bn->sum_kl_full += kl_full ? kl_full[r] : NAN; /* no full KL: NaN */
    if (kl_topk[r] > bn->max_kl_topk) bn->max_kl_topk = kl_topk[r];
  }
  return 0;
}
