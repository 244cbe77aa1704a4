/*
 * synth.c -- seeded synthetic logit rows shaped like the workloads of the
 * logit-diffing method (teacher-forced positions x full vocabulary).
 *
 * This module only PRODUCES inputs.  It holds none of the comparison
 * arithmetic (no softmax, KL, selection, margin or ULP statistics), so the
 * HIP path and the oracle can both be fed from it without sharing any of the
 * method's code.
 *
 * Random numbers: a counter-based use of SplitMix64 (Steele, Lea, Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014): output for
 * counter c under key k is mix64(k + (c + 1) * GAMMA), mix64 being the
 * published SplitMix64 output function.  Uniforms are 53-bit doubles in
 * (0, 1]; normals come from the Box-Muller transform (Box & Muller 1958) in
 * double precision, so |Z| <= sqrt(-2 ln 2^-53) ~= 8.572 for every draw.
 * bf16 values are produced by IEEE round-to-nearest-even from fp32.
 *
 * Every value depends only on (seed, stream, row, column), never on the
 * thread count or the block of rows requested, so any row range can be
 * regenerated on its own.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ull

enum {
  ST_BASE = 1,   /* baseline noise */
  ST_CAND = 2,   /* candidate noise */
  ST_ROW = 3,    /* per-row parameters (boost token and amount) */
  ST_SWAP = 4,   /* constructed top-2 rows */
  ST_PICK = 5,   /* subset selection hashes */
  ST_STEP = 6,   /* ULP step sizes */
};

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return mix64(seed * GAMMA + mix64(stream + GAMMA));
}

uint64_t synth_u64(uint64_t key, uint64_t ctr) { return mix64(key + (ctr + 1) * GAMMA); }

/* uniform double in (0, 1] */
static inline double unif(uint64_t key, uint64_t ctr) {
  return (double)((synth_u64(key, ctr) >> 11) + 1) * (1.0 / 9007199254740992.0);
}

/* standard normal for (row, col) of a row-major [*, cols] stream */
static inline double normal_at(uint64_t key, int64_t row, int64_t col, int64_t cols) {
  const int64_t pairs = (cols + 1) / 2;
  const uint64_t p = (uint64_t)(row * pairs + col / 2);
  const double u1 = unif(key, 2 * p), u2 = unif(key, 2 * p + 1);
  const double r = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586 * u2;
  double sn, cs;
  sincos(th, &sn, &cs);
  return (col & 1) ? r * sn : r * cs;
}

/* both normals of a pair at once (cols must be even, col even) */
static inline void normal_pair(uint64_t key, int64_t row, int64_t col, int64_t cols, double *z0,
                               double *z1) {
  const int64_t pairs = (cols + 1) / 2;
  const uint64_t p = (uint64_t)(row * pairs + col / 2);
  const double u1 = unif(key, 2 * p), u2 = unif(key, 2 * p + 1);
  const double r = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586 * u2;
  double sn, cs;
  sincos(th, &sn, &cs);
  *z0 = r * cs;
  *z1 = r * sn;
}

/* all normals of one row of a [*, cols] stream, pairwise (same values as normal_at) */
static void row_normals(uint64_t key, int64_t row, int64_t cols, double *z) {
  int64_t c = 0;
  for (; c + 1 < cols; c += 2) normal_pair(key, row, c, cols, &z[c], &z[c + 1]);
  if (c < cols) z[c] = normal_at(key, row, c, cols);
}

static inline uint32_t f2u(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
static inline float u2f(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* IEEE binary32 -> bfloat16, round to nearest, ties to even; NaN -> quiet NaN */
uint16_t synth_bf16_rne(float f) {
  uint32_t u = f2u(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

/* token index in [0, v) from a 64-bit draw (multiply-shift on the top 32 bits) */
static inline int64_t pick_token(uint64_t x, int64_t v) {
  return (int64_t)(((x >> 32) * (uint64_t)v) >> 32);
}

/* Per-row parameters shared by the logit-row configs: the boosted token and
 * the boost amount drawn from U[lo, hi]. */
static inline void row_boost(uint64_t seed, int64_t row, int64_t v, double lo, double hi,
                             int64_t *tok, double *amt) {
  const uint64_t k = synth_key(seed, ST_ROW);
  *tok = pick_token(synth_u64(k, 2 * (uint64_t)row), v);
  *amt = lo + (hi - lo) * unif(k, 2 * (uint64_t)row + 1);
}

/* ---------------------------------------------------------------------------------
 * Tiny compare: a = 2 Z + peak (U[0,8] on one random token), b = a + 0.05 Z'.  fp32.
 */
void synth_tiny(uint64_t seed, int64_t r0, int64_t nr, int64_t v, float *a, float *b) {
  const uint64_t ka = synth_key(seed, ST_BASE), kb = synth_key(seed, ST_CAND);
#pragma omp parallel
  {
    double *za = (double *)malloc((size_t)v * sizeof(double));
    double *zb = (double *)malloc((size_t)v * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t i = 0; i < nr; i++) {
      const int64_t r = r0 + i;
      int64_t tok;
      double amt;
      row_boost(seed, r, v, 0.0, 8.0, &tok, &amt);
      row_normals(ka, r, v, za);
      row_normals(kb, r, v, zb);
      float *ar = a + i * v, *br = b + i * v;
      for (int64_t c = 0; c < v; c++) {
        double x = 2.0 * za[c];
        if (c == tok) x += amt;
        ar[c] = (float)x;
        br[c] = (float)((double)ar[c] + 0.05 * zb[c]);
      }
    }
    free(za);
    free(zb);
  }
}

/* One "code-like" or "prose-like" baseline row in fp32:
 * x = 1.5 Z, plus a boost U[4,12] (code) or U[0,2] (prose) on one random token. */
static void logit_row(uint64_t seed, int64_t r, int64_t v, int code, double *z, float *out) {
  const uint64_t ka = synth_key(seed, ST_BASE);
  int64_t tok;
  double amt;
  row_boost(seed, r, v, code ? 4.0 : 0.0, code ? 12.0 : 2.0, &tok, &amt);
  row_normals(ka, r, v, z);
  for (int64_t c = 0; c < v; c++) out[c] = (float)(1.5 * z[c]);
  out[tok] = (float)((double)out[tok] + amt);
}

/* ---------------------------------------------------------------------------------
 * Decoded segment: fp32 both sides.  Even rows code-like, odd rows prose-like.
 * b = fp32(bf16_rne(a)).
 */
void synth_segment(uint64_t seed, int64_t r0, int64_t nr, int64_t v, float *a, float *b) {
#pragma omp parallel
  {
    double *z = (double *)malloc((size_t)v * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t i = 0; i < nr; i++) {
      const int64_t r = r0 + i;
      float *ar = a + i * v, *br = b + i * v;
      logit_row(seed, r, v, (r % 2) == 0, z, ar);
      for (int64_t c = 0; c < v; c++) br[c] = bf16_to_f32(synth_bf16_rne(ar[c]));
    }
    free(z);
  }
}

/* ---------------------------------------------------------------------------------
 * Scored-corpus rows: row r = depth*2048 + segment*512 + position; segments 0-1
 * code-like, 2-3 prose-like.  Baseline fp32, candidate bf16(a + 0.02 Z').
 * Rows flagged in `swap` (0/1 per row of the block) are built with a known top-2:
 * every token keeps 1.5 Z (so |x| <= 12.86), token t2 gets 13 + 2U and token t1
 * gets x[t2] + 1.25 + 2.75U' (a top-1/top-2 gap above 1.25); after the noise and
 * rounding the candidate values at t1 and t2 are exchanged.
 */
void synth_corpus(uint64_t seed, int64_t r0, int64_t nr, int64_t v, const uint8_t *swap, float *a,
                  uint16_t *b) {
  const uint64_t ka = synth_key(seed, ST_BASE), kb = synth_key(seed, ST_CAND);
  const uint64_t ks = synth_key(seed, ST_SWAP);
#pragma omp parallel
  {
    double *z = (double *)malloc((size_t)v * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t i = 0; i < nr; i++) {
      const int64_t r = r0 + i;
      const int code = ((r / 512) % 4) < 2;
      float *ar = a + i * v;
      uint16_t *br = b + i * v;
      int64_t t1 = -1, t2 = -1;
      if (swap && swap[i]) {
        row_normals(ka, r, v, z);
        for (int64_t c = 0; c < v; c++) ar[c] = (float)(1.5 * z[c]);
        t1 = pick_token(synth_u64(ks, 4 * (uint64_t)r), v);
        t2 = pick_token(synth_u64(ks, 4 * (uint64_t)r + 1), v - 1);
        if (t2 >= t1) t2++;
        const double top2 = 13.0 + 2.0 * unif(ks, 4 * (uint64_t)r + 2);
        const double top1 = top2 + 1.25 + 2.75 * unif(ks, 4 * (uint64_t)r + 3);
        ar[t2] = (float)top2;
        ar[t1] = (float)top1;
      } else {
        logit_row(seed, r, v, code, z, ar);
      }
      row_normals(kb, r, v, z);
      for (int64_t c = 0; c < v; c++)
        br[c] = synth_bf16_rne((float)((double)ar[c] + 0.02 * z[c]));
      if (t1 >= 0) {
        const uint16_t t = br[t1];
        br[t1] = br[t2];
        br[t2] = t;
      }
    }
    free(z);
  }
}

/* ---------------------------------------------------------------------------------
 * Large stream: both sides bf16.  a = bf16(code/prose row as in synth_segment),
 * b = bf16(fp32(a + 0.01 Z')).
 */
void synth_stream(uint64_t seed, int64_t r0, int64_t nr, int64_t v, uint16_t *a, uint16_t *b) {
  const uint64_t kb = synth_key(seed, ST_CAND);
#pragma omp parallel
  {
    float *row = (float *)malloc((size_t)v * sizeof(float));
    double *z = (double *)malloc((size_t)v * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t i = 0; i < nr; i++) {
      const int64_t r = r0 + i;
      uint16_t *ar = a + i * v, *br = b + i * v;
      logit_row(seed, r, v, (r % 2) == 0, z, row);
      row_normals(kb, r, v, z);
      for (int64_t c = 0; c < v; c++) {
        const uint16_t h = synth_bf16_rne(row[c]);
        ar[c] = h;
        br[c] = synth_bf16_rne((float)((double)bf16_to_f32(h) + 0.01 * z[c]));
      }
    }
    free(row);
    free(z);
  }
}

/* ---------------------------------------------------------------------------------
 * Bitwise sweep inputs.
 */

/* bf16(Z) rows of a [rows, cols] tensor */
void synth_bf16_normal(uint64_t seed, int64_t r0, int64_t nr, int64_t cols, uint16_t *a) {
  const uint64_t ka = synth_key(seed, ST_BASE);
#pragma omp parallel
  {
    double *z = (double *)malloc((size_t)cols * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t i = 0; i < nr; i++) {
      row_normals(ka, r0 + i, cols, z);
      for (int64_t c = 0; c < cols; c++) a[i * cols + c] = synth_bf16_rne((float)z[c]);
    }
    free(z);
  }
}

/* fp32 logit rows shaped like synth_segment's baseline */
void synth_logit_rows(uint64_t seed, int64_t r0, int64_t nr, int64_t v, float *a) {
#pragma omp parallel
  {
    double *z = (double *)malloc((size_t)v * sizeof(double));
#pragma omp for schedule(static)
    for (int64_t i = 0; i < nr; i++) logit_row(seed, r0 + i, v, ((r0 + i) % 2) == 0, z, a + i * v);
    free(z);
  }
}

/* 64-bit selection hash of flat position p: the m positions with the smallest
 * hashes form a uniform random m-subset (ties have probability ~2^-64). */
void synth_pick_hash(uint64_t seed, uint64_t stream, int64_t p0, int64_t np, uint64_t *out) {
  const uint64_t k = synth_key(seed, ST_PICK * 1000 + stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < np; i++) out[i] = synth_u64(k, (uint64_t)(p0 + i));
}

/* ULP step for the j-th injected position: +-1, +-2 or +-3 */
int synth_ulp_step(uint64_t seed, int64_t j) {
  const uint64_t x = synth_u64(synth_key(seed, ST_STEP), (uint64_t)j);
  const int mag = 1 + (int)((x >> 32) % 3u);
  return (x & 1u) ? -mag : mag;
}

/* Move a value by `step` units in the monotone integer ordering of the format
 * (width 16 = bf16, 32 = fp32): ordering o(u) = u | signbit for positive
 * patterns and ~u for negative ones.  Used only to build perturbed inputs. */
uint32_t synth_ulp_move(uint32_t u, int step, int width) {
  const uint32_t sign = width == 16 ? 0x8000u : 0x80000000u;
  const uint32_t all = width == 16 ? 0xffffu : 0xffffffffu;
  uint32_t o = (u & sign) ? (~u & all) : (u | sign);
  o = (uint32_t)((int64_t)o + step) & all;
  return (o & sign) ? (o & ~sign & all) : (~o & all);
}

/* Apply steps to a flat array of patterns at the given positions (in place). */
void synth_apply_ulp(void *data, int width, const int64_t *pos, const int32_t *step, int64_t m) {
  for (int64_t j = 0; j < m; j++) {
    if (width == 16) {
      uint16_t *d = (uint16_t *)data;
      d[pos[j]] = (uint16_t)synth_ulp_move(d[pos[j]], step[j], 16);
    } else {
      uint32_t *d = (uint32_t *)data;
      d[pos[j]] = synth_ulp_move(d[pos[j]], step[j], 32);
    }
  }
}

/* One row of standard normals from an arbitrary stream (for Monte-Carlo inputs). */
void synth_normals(uint64_t seed, uint64_t stream, int64_t row, int64_t n, double *out) {
  row_normals(synth_key(seed, stream), row, n, out);
}
