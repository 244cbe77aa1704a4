/*
 * lcmp.h -- C ABI of the teacher-forced logit comparison library (liblcmp.so,
 * HIP kernels for AMD CDNA4 / gfx950).
 *
 * The method is the one of the page "在 agent 时代如何快速验证 kernel 对精度的影响"
 * (susun-blog, verify-kernel-precision-with-logits; cited below as [logits]):
 * feed the same fixed text to a ground-truth implementation (the baseline)
 * and to the implementation under test (the candidate), record at every
 * position the next-token logits over the full vocabulary, and compare the two
 * distributions row by row (section 看 logits，而不是 token, teacher forcing).
 * The bitwise statistics follow the full-logit integer compare of the page
 * "Kestrel_VLLM - 18 · 投机解码位级对拍收口" (section 二; cited as [bitexact]) and the
 * arithmetic layer of the correctness ladder on the page "海光 DCU 实测：BF16
 * 逐位一致为什么仍可能出现文本漂移" (sections 1 and 7; cited as [dcu]).
 *
 * Conventions shared by every entry point
 *   - Tensors are row-major [rows, ld] with ld >= the number of columns used;
 *     leading dimensions count elements.  Element types: LCMP_F32 (IEEE
 *     binary32) or LCMP_BF16 (bfloat16 bit patterns, uint16 storage).
 *   - Every data pointer (inputs, outputs, workspace) is DEVICE memory on the
 *     current HIP device, except the lcmp_row_out struct itself and `edges`,
 *     which are host memory read during the call.
 *   - The caller owns every buffer.  The library allocates and frees nothing,
 *     keeps no mutable global state, is reentrant, and calls on different
 *     streams may run concurrently if their workspaces differ.  A call enqueues
 *     kernels only (no memset, no copy), so it can be captured in a HIP graph
 *     and replayed on new contents of the same buffers.  The one exception is
 *     lcmp_compare_logits_noalloc, whose workspace is a fixed array the library
 *     holds on each device (see there).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and is asynchronous: results are valid once the caller has
 *     synchronised with that stream.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     negative return nothing has been launched and no output was written.
 *     A launch failure returns LCMP_EHIP.  The library never aborts, exits
 *     or prints.
 *   - Results are deterministic: the same inputs, sizes and flags give
 *     bit-identical outputs on every run (fixed-order reductions, no floating
 *     atomics).
 */
#ifndef LCMP_H
#define LCMP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCMP_ABI_VERSION 4
#define LCMP_MAX_K 64       /* largest top-k */
#define LCMP_MAX_EDGES 32   /* largest number of margin-bin edges */
#define LCMP_MAX_GROUPS 256 /* largest number of row groups in lcmp_bin_report */
#define LCMP_MAX_BINS 256   /* largest n_groups * n_edges */
#define LCMP_MAX_ROWS 2147483647LL /* largest n (rows) of the compare, bitwise and record calls */

typedef enum { LCMP_F32 = 0, LCMP_BF16 = 1 } lcmp_dtype;

typedef enum {
  LCMP_OK = 0,
  LCMP_EINVAL = -1,     /* NULL required pointer, negative count, bad flag, misaligned workspace */
  LCMP_EDTYPE = -2,     /* unknown element type */
  LCMP_ESHAPE = -3,     /* v < 2, k out of [1, LCMP_MAX_K], ld < columns, n > LCMP_MAX_ROWS, bin counts too large */
  LCMP_EWORKSPACE = -4, /* workspace NULL or smaller than the matching *_workspace_bytes() */
  LCMP_EHIP = -5,       /* a HIP launch or runtime call failed */
  LCMP_EEDGES = -6      /* edges not strictly ascending, not positive, NaN, or too many */
} lcmp_status;

/* flags of lcmp_compare_logits */
#define LCMP_WITH_BITDIFF 1u /* also fill per-row bitwise statistics in the same pass */

/* per-row status bits (lcmp_row_out.status) */
#define LCMP_ROW_NONFINITE 1u /* a NaN or +inf on either side */
#define LCMP_ROW_EMPTY 2u     /* the baseline or the candidate row is entirely -inf */

/*
 * Per-position outputs of lcmp_compare_logits: device arrays of n entries
 * (topk_idx: n*k).  Any pointer may be NULL to skip that output.
 *
 *   kl_full   KL(P||Q) = sum_i p_i ln(p_i / q_i) over the full vocabulary, P the
 *             baseline softmax and Q the candidate softmax at temperature 1
 *             ([logits] 怎么比两个分布, KL equation).  +inf when some p_i > 0 has
 *             q_i = 0 (candidate -inf where the baseline is finite).
 *   kl_topk   KL over the baseline's top-k tokens plus one "other" bucket holding
 *             the rest of the mass on each side ([logits] 怎么比两个分布, top-20
 *             paragraph).  Equals kl_full when k >= v - 1.
 *   margin    baseline top-1 logit minus top-2 logit, one double subtraction
 *             ([logits] 怎么比两个分布, margin paragraph).
 *   lse_base, lse_cand   log of each side's softmax normaliser.
 *   top1_base, top2_base baseline's two largest logits, lower index first on ties.
 *   top1_cand candidate's largest logit, lowest index on ties.
 *   flip      1 when top1_cand != top1_base ([logits] 怎么比两个分布, top-1 flip).
 *   topk_idx  the baseline's k largest logits, value descending, index ascending;
 *             entries past min(k, v) are -1.
 *   status    0 or a mask of LCMP_ROW_* bits.  A flagged row reports NaN in the
 *             double fields, -1 in the index fields and 0 in flip.
 *   target    optional INPUT, device [n]: the teacher-forced next token of each
 *             position (the token the fixed text continues with).
 *   logp_base, logp_cand   ln p(target) = a[target] - lse_base and
 *             ln q(target) = b[target] - lse_cand, the only numbers perplexity
 *             looks at ([logits] perplexity（困惑度）看不出这一级的差别).  Require
 *             target; a target outside [0, v) or a flagged row gives NaN.
 */
typedef struct {
  double *kl_topk, *kl_full, *margin, *lse_base, *lse_cand;
  int32_t *top1_base, *top2_base, *top1_cand;
  uint8_t *flip, *status;
  int32_t *topk_idx;
  const int32_t *target;
  double *logp_base, *logp_cand;
} lcmp_row_out;

/*
 * Per-row bitwise statistics ([bitexact] 二: compare full rows as integers,
 * report the number of differing elements and the first nonzero-ULP position;
 * [dcu] §1, §7: finite check, max abs, mean abs, relative L2, mismatch count).
 *
 *   ndiff        elements whose bit patterns differ
 *   first_diff   lowest such column, -1 if none
 *   max_ulp      largest |o(a) - o(b)| with o(u) = u | signbit for a clear sign bit
 *                and ~u otherwise (a monotone integer image; +0 and -0 are 1 apart)
 *   nonfinite_a, nonfinite_b   NaN / +-inf elements on each side
 *   max_abs, sum_abs, sum_sq_diff, sum_sq_base   over columns where both values
 *                are finite: max |a-b|, sum |a-b|, sum (a-b)^2, sum a^2
 *   mean_abs     sum_abs / cols
 *   rel_l2       sqrt(sum_sq_diff / sum_sq_base); 0 if both sums are 0, +inf if
 *                only sum_sq_base is 0
 * Same element type on both sides: patterns compared at that width (16 or 32
 * bits).  Mixed types: bf16 widened exactly to fp32 patterns, compared at 32.
 */
typedef struct {
  int64_t ndiff, first_diff, nonfinite_a, nonfinite_b;
  uint32_t max_ulp, pad_;
  double max_abs, sum_abs, sum_sq_diff, sum_sq_base, mean_abs, rel_l2;
} lcmp_bitdiff_row;

/* One margin bin of one group ([logits] 三者联合起来验证精度问题: flips counted per
 * margin bin).  max_kl_topk is -inf for an empty bin. */
typedef struct {
  int64_t count, flips, ties, tie_flips;
  double sum_kl_topk, sum_kl_full, max_kl_topk;
} lcmp_bin;

/* Per-group totals: flips at margin strictly above the big-margin threshold (the
 * page's stop rule uses 1), rows excluded by a nonzero status, rows whose margin
 * lies in no bin. */
typedef struct {
  int64_t big_margin_flips, excluded, unbinned;
} lcmp_group_summary;

int lcmp_abi_version(void);
const char *lcmp_strerror(int status);

/* ---------------------------------------------------------------- compare */

/* Workspace bytes that lcmp_compare_logits needs for these sizes and flags
 * (0 on invalid sizes).  The workspace must be 16-byte aligned. */
size_t lcmp_compare_workspace_bytes(int64_t n, int64_t v, int k, uint32_t flags);

/* The same query under the short name of the problem statement's interface:
 * identical arguments and result. */
size_t lcmp_workspace_bytes(int64_t n, int64_t v, int k, uint32_t flags);

/*
 * Compare n teacher-forced positions: baseline row i against candidate row i,
 * the first v columns of each ([logits] 看 logits，而不是 token and 怎么比两个分布).
 *   base, cand    device, [n, ld_base] of type tb and [n, ld_cand] of type tc; the
 *                 two types may differ.
 *   k             top-k size, 1..LCMP_MAX_K (the page uses 20); v >= 2.
 *   flags         0 or LCMP_WITH_BITDIFF; with it, bd (device [n]) receives the
 *                 bitwise statistics of each row pair (bd may be NULL otherwise).
 *   out           host struct of device output pointers (see lcmp_row_out).
 * One pass reads each row pair once.  Rows whose "other"-bucket term is
 * ill-conditioned in the one-pass sums (the candidate keeps nearly all of its
 * mass inside the baseline's top-k) have their two buckets summed again
 * directly by the wave that finishes the row, so such rows read their pair
 * once more; ordinary rows never are.
 * With n == 0 nothing is launched and no row, output or workspace pointer is
 * read (they may be NULL).
 * Returns LCMP_OK or a negative lcmp_status.
 */
int lcmp_compare_logits(const void *base, int tb, int64_t ld_base, const void *cand, int tc,
                        int64_t ld_cand, int64_t n, int64_t v, int k, uint32_t flags,
                        const lcmp_row_out *out, lcmp_bitdiff_row *bd, void *workspace,
                        size_t ws_bytes, void *stream);

/*
 * Instrumented form of lcmp_compare_logits for measuring the streaming pass:
 * ev_before / ev_after (hipEvent_t created with timing, or NULL) are given to
 * the dispatch of the streaming kernel (hipExtLaunchKernel), so they take its
 * start and end time and their elapsed time is that kernel's duration.  With
 * n == 0 nothing is launched and both are recorded on `stream` back to back.
 * Everything else is identical.
 */
int lcmp_compare_logits_timed(const void *base, int tb, int64_t ld_base, const void *cand, int tc,
                              int64_t ld_cand, int64_t n, int64_t v, int k, uint32_t flags,
                              const lcmp_row_out *out, lcmp_bitdiff_row *bd, void *workspace,
                              size_t ws_bytes, void *stream, void *ev_before, void *ev_after);

/*
 * Allocation-free form of lcmp_compare_logits, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc.  Identical arguments and results,
 * minus the workspace: the call uses a scratch array of
 * LCMP_NOALLOC_SCRATCH_BYTES that the library keeps in device memory on each
 * device it runs on until the process ends (its address is looked up once per
 * device, on the first call there).  The caller still owns inputs and outputs.
 * The call allocates and frees nothing.
 *   Limits: sizes whose workspace (lcmp_compare_workspace_bytes(n, v, k, flags))
 *   exceeds LCMP_NOALLOC_SCRATCH_BYTES return LCMP_EWORKSPACE, before anything
 *   is launched (at V = 151936, k = 20 with bitwise statistics every n up to
 *   73728 fits); split larger batches into row ranges.  LCMP_EHIP if the
 *   array's address cannot be obtained.  Other errors as lcmp_compare_logits.
 *   Every call on a device shares that device's array: calls that overlap in
 *   time on one device (two streams, two threads) race and give wrong results;
 *   serialise them.  Nothing needs clearing between calls (the kernels
 *   initialise what they read).
 */
#define LCMP_NOALLOC_SCRATCH_BYTES (64ull << 20) /* 64 MiB per device */
int lcmp_compare_logits_noalloc(const void *base, int tb, int64_t ld_base, const void *cand,
                                int tc, int64_t ld_cand, int64_t n, int64_t v, int k,
                                uint32_t flags, const lcmp_row_out *out, lcmp_bitdiff_row *bd,
                                void *stream);

/* ---------------------------------------------------------------- bitwise */

size_t lcmp_bitdiff_workspace_bytes(int64_t rows, int64_t cols);

/*
 * Bitwise / ULP statistics of a [rows, cols] pair (see lcmp_bitdiff_row).
 *   a, b   device, [rows, lda] of type ta and [rows, ldb] of type tb.
 *   out    device [rows].
 */
int lcmp_bitdiff(const void *a, int ta, int64_t lda, const void *b, int tb, int64_t ldb,
                 int64_t rows, int64_t cols, lcmp_bitdiff_row *out, void *workspace,
                 size_t ws_bytes, void *stream);

/* Instrumented form of lcmp_bitdiff: ev_before / ev_after (hipEvent_t, may be
 * NULL) take the start and end time of the streaming kernel's dispatch, as in
 * lcmp_compare_logits_timed. */
int lcmp_bitdiff_timed(const void *a, int ta, int64_t lda, const void *b, int tb, int64_t ldb,
                       int64_t rows, int64_t cols, lcmp_bitdiff_row *out, void *workspace,
                       size_t ws_bytes, void *stream, void *ev_before, void *ev_after);

/* ---------------------------------------------------------------- perturbations */

/* modes of lcmp_perturb */
#define LCMP_PERTURB_MANTISSA 0   /* keep `param` (0..23) fraction bits, fp32 exponent range */
#define LCMP_PERTURB_E4M3 1       /* fp8 e4m3 (fn): 3 fraction bits, largest 448, saturating */
#define LCMP_PERTURB_E4M3_SCALED 2 /* e4m3(x * 448) / 448, product and quotient in fp32 */

/*
 * Precision perturbations for precision-knee experiments ([logits] 实验 section:
 * cut a tensor's precision a step at a time -- keep only m fraction bits with
 * the exponent range unchanged, or round to fp8 e4m3 directly or after scaling
 * by 448 -- and watch where the KL starts to rise).  Elementwise:
 *   dst[r, c] = perturb(src[r, c]),  r < rows, c < cols.
 * Rounding is to nearest, ties to even; NaN stays NaN; a value rounded past
 * the largest fp32 becomes inf (mantissa mode) or 448 (e4m3 modes).  bf16
 * rounding is LCMP_PERTURB_MANTISSA with param 7.
 *   src    device [rows, ld_src] of type ts (fp32 or bf16, widened exactly).
 *   dst    device [rows, ld_dst] of type td; bf16 only when every result is a
 *          bf16 value (mantissa mode with param <= 7, or LCMP_PERTURB_E4M3),
 *          else LCMP_EDTYPE.  dst may be src when ts == td and ld_src == ld_dst.
 * Errors: LCMP_EINVAL for an unknown mode, a param outside 0..23 or a NULL
 * buffer; LCMP_ESHAPE for ld < cols or sizes too large.
 */
int lcmp_perturb(const void *src, int ts, int64_t ld_src, void *dst, int td, int64_t ld_dst,
                 int64_t rows, int64_t cols, int mode, int param, void *stream);

/* ---------------------------------------------------------------- compact record */

/*
 * A compact record of baseline rows ([logits] 先要有一个 ground truth: run the
 * ground truth once over the fixed text, store its distributions, and compare
 * every later change against that store rather than against the previous
 * version).  Per row it keeps what the top-k + "other" comparison needs:
 *   topk_idx     device [n, k_rec]: the k_rec largest logits' columns, value
 *                descending, index ascending; -1 past min(k_rec, v)
 *   topk_val     device [n, k_rec]: those logits (bf16 widened exactly); -inf
 *                past min(k_rec, v)
 *   lse_rest     device [n]: ln of the sum of exp(logit) over every other
 *                column; -inf when nothing is left
 *   status       device [n]: LCMP_ROW_NONFINITE / LCMP_ROW_EMPTY of the baseline
 *                row alone; a flagged row holds -1 / NaN in the fields above
 *   logp_target  device [n] or NULL: ln p(target) of the baseline, filled when
 *                the record is made with targets
 * At k_rec = 20 a row takes 169 bytes (177 with logp_target), against 4 v bytes
 * of an fp32 row.  Records are plain arrays: the caller stores and reloads them.
 */
typedef struct {
  int32_t *topk_idx;
  float *topk_val;
  double *lse_rest;
  uint8_t *status;
  double *logp_target;
} lcmp_record;

/* Workspace bytes of lcmp_record_baseline (0 on invalid sizes). */
size_t lcmp_record_workspace_bytes(int64_t n, int64_t v, int k_rec);

/*
 * Make the record of n baseline rows (the first v columns of each).
 *   base     device [n, ld_base] of type tb.
 *   k_rec    entries per row, 2..LCMP_MAX_K (a comparison may use any k <= k_rec).
 *   target   device [n] or NULL; required when rec->logp_target is set.  A target
 *            outside [0, v) gives NaN.
 *   rec      host struct of device arrays, filled by the call.
 * Errors: LCMP_ESHAPE for k_rec outside [2, LCMP_MAX_K], v < 2 or ld_base < v;
 * LCMP_EINVAL for a NULL array or logp_target without target.
 */
int lcmp_record_baseline(const void *base, int tb, int64_t ld_base, int64_t n, int64_t v,
                         int k_rec, const int32_t *target, const lcmp_record *rec,
                         void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes of lcmp_compare_record (0 on invalid sizes). */
size_t lcmp_compare_record_workspace_bytes(int64_t n, int64_t v);

/*
 * Compare n candidate rows against a record made with k_rec entries per row,
 * using its first k (1 <= k <= k_rec): reads the record and the candidate only,
 * so half the bytes of lcmp_compare_logits for equal element types.
 *   out   as for lcmp_compare_logits, with the same definitions, except:
 *         kl_full must be NULL (it needs the whole baseline row; LCMP_EINVAL
 *         otherwise); logp_base is the record's logp_target (LCMP_EINVAL when the
 *         record has none); lse_base is rebuilt from the record.
 * The status is LCMP_ROW_NONFINITE when the record row or the candidate row is,
 * else LCMP_ROW_EMPTY when either is.  The record must come from
 * lcmp_record_baseline with the same v; its entries are only read.
 */
int lcmp_compare_record(const lcmp_record *rec, int k_rec, const void *cand, int tc,
                        int64_t ld_cand, int64_t n, int64_t v, int k, const lcmp_row_out *out,
                        void *workspace, size_t ws_bytes, void *stream);

/* Instrumented form: ev_before / ev_after (hipEvent_t, may be NULL) take the
 * start and end time of the candidate's streaming kernel, as in
 * lcmp_compare_logits_timed. */
int lcmp_compare_record_timed(const lcmp_record *rec, int k_rec, const void *cand, int tc,
                              int64_t ld_cand, int64_t n, int64_t v, int k,
                              const lcmp_row_out *out, void *workspace, size_t ws_bytes,
                              void *stream, void *ev_before, void *ev_after);

/* ---------------------------------------------------------------- margin bins */

#define LCMP_MAX_BIN_ROWS (1LL << 36) /* largest n of lcmp_bin_report */

/* Workspace of lcmp_bin_report for n rows; 0 when n, n_groups or n_edges are
 * out of range. */
size_t lcmp_bin_workspace_bytes(int64_t n, int n_groups, int n_edges);

/*
 * Flip counts and KL sums per margin bin and group ([logits] 三者联合起来验证精度
 * 问题: bin flips by margin, compare each bin with the normal difference, and
 * treat a flip at a large margin as a stop).
 *   margin, flip, kl_topk, kl_full   device [n], typically lcmp_compare_logits output;
 *            kl_full may be NULL (a comparison against a record has none), and
 *            then sum_kl_full is NaN in every bin that holds a row.
 *   status   device [n] or NULL; rows with a nonzero status count as `excluded`.
 *   group    device [n] or NULL (all rows in group 0); ids outside [0, n_groups)
 *            are skipped.
 *   edges    HOST [n_edges], strictly ascending, positive, the last may be +inf.
 *            Bin j holds margins in [edges[j-1], edges[j]) with edges[-1] = 0.
 *   big_margin   threshold of the stop rule (the page uses 1): a flip with
 *            margin > big_margin is counted in big_margin_flips.
 *   bins     device [n_groups * n_edges]; summary device [n_groups].
 * n above LCMP_MAX_BIN_ROWS returns LCMP_ESHAPE.  Sums are formed in a fixed
 * order, so repeated calls are bit-identical.
 */
int lcmp_bin_report(const double *margin, const uint8_t *flip, const double *kl_topk,
                    const double *kl_full, const uint8_t *status, const int32_t *group,
                    int n_groups, int64_t n, const double *edges, int n_edges, double big_margin,
                    lcmp_bin *bins, lcmp_group_summary *summary, void *workspace,
                    size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- measurement */

/*
 * Read-only reference stream for measurement, not part of the comparison: it
 * reads the first v columns of the n row pairs exactly as lcmp_compare_logits
 * streams them (the same chunks of each row, steps of 512 elements of each
 * side, the same 8-byte or 16-byte non-temporal loads per lane, the next
 * step's loads in flight) and only XORs the words, so its duration is the
 * read time this access pattern reaches on the device.  One 32-bit word per
 * (row, chunk) is written to the workspace, which must hold at least
 * lcmp_compare_workspace_bytes(n, v, 1, 0) bytes.  ev_before / ev_after
 * (hipEvent_t, may be NULL) take the start and end time of the kernel, as in
 * lcmp_compare_logits_timed.
 * Errors as lcmp_compare_logits; LCMP_EINVAL also when a row start of either
 * tensor is not 16-byte aligned (the comparison then takes its scalar-load path).
 */
int lcmp_read_probe(const void *base, int tb, int64_t ld_base, const void *cand, int tc,
                    int64_t ld_cand, int64_t n, int64_t v, void *workspace, size_t ws_bytes,
                    void *stream, void *ev_before, void *ev_after);

#ifdef __cplusplus
}
#endif

#endif /* LCMP_H */
