// lcmp_api.hip -- the C ABI of liblcmp: argument checks, workspace layout,
// chunking, launches.  Declarations and the contract live in include/lcmp.h.
#include "../../include/lcmp.h"

#include <math.h>
#include <string.h>

#include <mutex>

#include "common.hpp"
#include "launch.hpp"

using namespace lcmp;

static_assert(sizeof(lcmp_bitdiff_row) == sizeof(BitdiffRow), "bitdiff row layout");
static_assert(sizeof(lcmp_bin) == sizeof(BinAcc), "bin layout");
static_assert(sizeof(lcmp_group_summary) == sizeof(GroupAcc), "group summary layout");
static_assert(kMaxGroups == LCMP_MAX_GROUPS && kMaxBins == LCMP_MAX_BINS &&
                  kMaxEdges == LCMP_MAX_EDGES && kMaxK == LCMP_MAX_K &&
                  kMaxBinRows == LCMP_MAX_BIN_ROWS,
              "limits of the header and of the kernels agree");

hipError_t lcmp::record_empty(const Timing &t, hipStream_t stream) {
  if (t.before && hipEventRecord(t.before, stream) != hipSuccess) return hipErrorUnknown;
  if (t.after && hipEventRecord(t.after, stream) != hipSuccess) return hipErrorUnknown;
  return hipSuccess;
}

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

Timing timing(void *ev_before, void *ev_after) {
  Timing t;
  t.before = (hipEvent_t)ev_before;
  t.after = (hipEvent_t)ev_after;
  return t;
}

// A call with no rows: nothing to launch, but the timing events of an
// instrumented call are still recorded (back to back).
int empty_call(void *ev_before, void *ev_after, void *stream) {
  return record_empty(timing(ev_before, ev_after), (hipStream_t)stream) == hipSuccess ? LCMP_OK
                                                                                      : LCMP_EHIP;
}

bool dtype_ok(int t) { return t == LCMP_F32 || t == LCMP_BF16; }
size_t esize(int t) { return t == LCMP_BF16 ? 2 : 4; }

// Chunks per row: enough (row, chunk) waves to fill the GPU several times over
// (256 CUs x 16 waves, four times), without cutting a row into pieces shorter
// than 16 wave steps.  A function of the sizes only, so the summation order,
// and hence every result bit, does not depend on the device or the stream.
struct Chunking {
  int64_t chunk;
  int32_t nchunks;
};

Chunking choose_chunks(int64_t n, int64_t v) {
  // Split rows into c chunks when there are too few rows to fill the chip.
  // Cost model: waves run in rounds of kResidentWaves (256 CUs x 16 waves);
  // a chunk of s steps costs s + kChunkOverheadSteps.  Among c in
  // [1, min(16, steps / 16)] take the cheapest, the smallest c on ties.  The
  // choice depends only on (n, v), so results are repeatable.
  constexpr int64_t kResidentWaves = 256 * 16;
  constexpr int64_t kChunkOverheadSteps = 2;
  const int64_t steps = (v + kSpan - 1) / kSpan;
  int64_t cmax = steps / 16;
  if (cmax > 16) cmax = 16;
  if (cmax < 1) cmax = 1;
  int64_t best_c = 1, best_cost = -1;
  for (int64_t c = 1; c <= cmax; ++c) {
    const int64_t rounds = n > 0 ? (n * c + kResidentWaves - 1) / kResidentWaves : 1;
    const int64_t cost = rounds * ((steps + c - 1) / c + kChunkOverheadSteps);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best_c = c;
    }
  }
  const int64_t per = (steps + best_c - 1) / best_c;
  Chunking ch;
  ch.chunk = per * kSpan;
  ch.nchunks = (int32_t)((v + ch.chunk - 1) / ch.chunk);
  return ch;
}

int kint_of(int64_t v, int k) {
  const int64_t keff = (int64_t)k < v ? (int64_t)k : v;
  return (int)(keff < 2 ? 2 : keff);
}

struct CompareLayout {
  Chunking ch;
  int kint;
  size_t off_stats, off_bits, off_ta, off_ti;
  size_t total;
};

CompareLayout compare_layout(int64_t n, int64_t v, int k, uint32_t flags) {
  CompareLayout L;
  L.ch = choose_chunks(n, v);
  L.kint = kint_of(v, k);
  const size_t items = (size_t)n * (size_t)L.ch.nchunks;
  size_t o = 0;
  L.off_stats = o;
  o = align_up(o + items * sizeof(ChunkStats));
  L.off_bits = o;
  if (flags & LCMP_WITH_BITDIFF) o = align_up(o + items * sizeof(ChunkBits));
  L.off_ta = o;
  o = align_up(o + items * (size_t)L.kint * sizeof(float));
  L.off_ti = o;
  o = align_up(o + items * (size_t)L.kint * sizeof(int32_t));
  L.total = o;
  return L;
}

// 16-byte loads need every row start of both tensors 16-byte aligned
bool vector_ok(const void *a, int ta, int64_t lda, const void *b, int tb, int64_t ldb) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  return pa % 16 == 0 && pb % 16 == 0 && ((size_t)lda * esize(ta)) % 16 == 0 &&
         ((size_t)ldb * esize(tb)) % 16 == 0;
}

// Chunks of the one-side pass of the record comparison: the same cost model
// as choose_chunks, in units of kRestChunkQuantum columns (two fp32 steps or
// one bf16 step of a wave), with at least four units per chunk.
struct RestLayout {
  Chunking ch;
  size_t bytes;
};

RestLayout rest_layout(int64_t n, int64_t v) {
  constexpr int64_t kResidentWaves = 256 * 16;
  constexpr int64_t kChunkOverhead = 1;
  const int64_t units = (v + kRestChunkQuantum - 1) / kRestChunkQuantum;
  int64_t cmax = units / 4;
  if (cmax > 16) cmax = 16;
  if (cmax < 1) cmax = 1;
  int64_t best_c = 1, best_cost = -1;
  for (int64_t c = 1; c <= cmax; ++c) {
    const int64_t rounds = n > 0 ? (n * c + kResidentWaves - 1) / kResidentWaves : 1;
    const int64_t cost = rounds * ((units + c - 1) / c + kChunkOverhead);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best_c = c;
    }
  }
  RestLayout L;
  L.ch.chunk = (units + best_c - 1) / best_c * kRestChunkQuantum;
  L.ch.nchunks = (int32_t)((v + L.ch.chunk - 1) / L.ch.chunk);
  L.bytes = align_up((size_t)n * (size_t)L.ch.nchunks * sizeof(RestChunk));
  return L;
}

bool rows_aligned(const void *p, int t, int64_t ld) {
  return (uintptr_t)p % 16 == 0 && ((size_t)ld * esize(t)) % 16 == 0;
}

bool record_ok(const lcmp_record *rec) {
  return rec->topk_idx && rec->topk_val && rec->lse_rest && rec->status;
}

constexpr int64_t kMaxCols = 0x7fffffffLL - 4096;  // indices are 32-bit in the kernels
// the per-row kernels launch one block per row, and a grid dimension holds
// at most 2^31 - 1 blocks
constexpr int64_t kMaxRows = LCMP_MAX_ROWS;

}  // namespace

extern "C" {

int lcmp_abi_version(void) { return LCMP_ABI_VERSION; }

const char *lcmp_strerror(int status) {
  switch (status) {
    case LCMP_OK: return "ok";
    case LCMP_EINVAL: return "invalid argument (null pointer, negative count, unknown flag or misaligned workspace)";
    case LCMP_EDTYPE: return "unknown element type";
    case LCMP_ESHAPE: return "invalid shape (v < 2, k outside [1, LCMP_MAX_K], ld < columns, or too large)";
    case LCMP_EWORKSPACE: return "workspace missing or too small";
    case LCMP_EHIP: return "HIP launch or runtime error";
    case LCMP_EEDGES: return "margin-bin edges invalid (must be positive, strictly ascending, at most LCMP_MAX_EDGES)";
    default: return "unknown status";
  }
}

size_t lcmp_compare_workspace_bytes(int64_t n, int64_t v, int k, uint32_t flags) {
  if (n < 0 || v < 2 || v > kMaxCols || n > kMaxRows || k < 1 || k > LCMP_MAX_K) return 0;
  if (n == 0) return kAlign;
  return compare_layout(n, v, k, flags).total;
}

size_t lcmp_workspace_bytes(int64_t n, int64_t v, int k, uint32_t flags) {
  return lcmp_compare_workspace_bytes(n, v, k, flags);
}

}  // extern "C"

static int compare_impl(const void *base, int tb, int64_t ld_base, const void *cand, int tc,
                        int64_t ld_cand, int64_t n, int64_t v, int k, uint32_t flags,
                        const lcmp_row_out *out, lcmp_bitdiff_row *bd, void *workspace,
                        size_t ws_bytes, void *stream, void *ev_before, void *ev_after) {
  if (!dtype_ok(tb) || !dtype_ok(tc)) return LCMP_EDTYPE;
  if (n < 0 || (flags & ~LCMP_WITH_BITDIFF) != 0 || !out) return LCMP_EINVAL;
  if (v < 2 || v > kMaxCols || n > kMaxRows || k < 1 || k > LCMP_MAX_K || ld_base < v ||
      ld_cand < v)
    return LCMP_ESHAPE;
  const bool with_bits = (flags & LCMP_WITH_BITDIFF) != 0;
  if ((out->logp_base || out->logp_cand) && !out->target) return LCMP_EINVAL;
  if (n == 0) return empty_call(ev_before, ev_after, stream);
  if (with_bits && !bd) return LCMP_EINVAL;
  if (!base || !cand) return LCMP_EINVAL;
  const CompareLayout L = compare_layout(n, v, k, flags);
  if (!workspace || ws_bytes < L.total) return LCMP_EWORKSPACE;
  if ((uintptr_t)workspace % 16 != 0) return LCMP_EINVAL;

  char *ws = (char *)workspace;
  StreamArgs sa;
  sa.a = base;
  sa.b = cand;
  sa.lda = ld_base;
  sa.ldb = ld_cand;
  sa.n = n;
  sa.v = v;
  sa.chunk = L.ch.chunk;
  sa.nchunks = L.ch.nchunks;
  sa.kint = L.kint;
  sa.stats = (ChunkStats *)(ws + L.off_stats);
  sa.bits = with_bits ? (ChunkBits *)(ws + L.off_bits) : nullptr;
  sa.ta = (float *)(ws + L.off_ta);
  sa.ti = (int32_t *)(ws + L.off_ti);
  hipStream_t s = (hipStream_t)stream;
  if (launch_row_stats(sa, tb, tc, true, with_bits, vector_ok(base, tb, ld_base, cand, tc, ld_cand),
                       s, timing(ev_before, ev_after)) != hipSuccess)
    return LCMP_EHIP;

  FinalArgs fa;
  fa.stats = sa.stats;
  fa.bits = sa.bits;
  fa.ta = sa.ta;
  fa.ti = sa.ti;
  fa.cand = cand;
  fa.tc = tc;
  fa.ldc = ld_cand;
  fa.base = base;
  fa.tb = tb;
  fa.ldb = ld_base;
  const bool with_target = out->target && (out->logp_base || out->logp_cand);
  fa.target = with_target ? out->target : nullptr;
  fa.logp_base = with_target ? out->logp_base : nullptr;
  fa.logp_cand = with_target ? out->logp_cand : nullptr;
  fa.n = n;
  fa.v = v;
  fa.nchunks = L.ch.nchunks;
  fa.kint = L.kint;
  fa.k = k;
  fa.kl_topk = out->kl_topk;
  fa.kl_full = out->kl_full;
  fa.margin = out->margin;
  fa.lse_base = out->lse_base;
  fa.lse_cand = out->lse_cand;
  fa.top1_base = out->top1_base;
  fa.top2_base = out->top2_base;
  fa.top1_cand = out->top1_cand;
  fa.flip = out->flip;
  fa.status = out->status;
  fa.topk_idx = out->topk_idx;
  fa.bd = with_bits ? (BitdiffRow *)bd : nullptr;
  if (launch_topk_kl(fa, s) != hipSuccess) return LCMP_EHIP;
  return LCMP_OK;
}

extern "C" {

int lcmp_compare_logits(const void *base, int tb, int64_t ld_base, const void *cand, int tc,
                        int64_t ld_cand, int64_t n, int64_t v, int k, uint32_t flags,
                        const lcmp_row_out *out, lcmp_bitdiff_row *bd, void *workspace,
                        size_t ws_bytes, void *stream) {
  return compare_impl(base, tb, ld_base, cand, tc, ld_cand, n, v, k, flags, out, bd, workspace,
                      ws_bytes, stream, nullptr, nullptr);
}

int lcmp_compare_logits_timed(const void *base, int tb, int64_t ld_base, const void *cand, int tc,
                              int64_t ld_cand, int64_t n, int64_t v, int k, uint32_t flags,
                              const lcmp_row_out *out, lcmp_bitdiff_row *bd, void *workspace,
                              size_t ws_bytes, void *stream, void *ev_before, void *ev_after) {
  return compare_impl(base, tb, ld_base, cand, tc, ld_cand, n, v, k, flags, out, bd, workspace,
                      ws_bytes, stream, ev_before, ev_after);
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free compare

// The workspace of lcmp_compare_logits_noalloc: one array per device, in
// device memory for as long as the library is loaded.  Its name is only a
// host-side stand-in for the symbol; host code uses the device address that
// hipGetSymbolAddress returns for the current device, kept per device below.
static __device__ __align__(256) unsigned char scratch[LCMP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, set once

// Device address of this device's scratch array (nullptr on a HIP error).
// The first call on a device looks the symbol up with that device current.
void *scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int lcmp_compare_logits_noalloc(const void *base, int tb, int64_t ld_base, const void *cand,
                                int tc, int64_t ld_cand, int64_t n, int64_t v, int k,
                                uint32_t flags, const lcmp_row_out *out, lcmp_bitdiff_row *bd,
                                void *stream) {
  // the size checks of compare_impl first, so a bad shape is reported as such
  if (!dtype_ok(tb) || !dtype_ok(tc)) return LCMP_EDTYPE;
  if (n < 0 || (flags & ~LCMP_WITH_BITDIFF) != 0 || !out) return LCMP_EINVAL;
  if (v < 2 || v > kMaxCols || n > kMaxRows || k < 1 || k > LCMP_MAX_K || ld_base < v ||
      ld_cand < v)
    return LCMP_ESHAPE;
  if (n == 0) return compare_impl(base, tb, ld_base, cand, tc, ld_cand, n, v, k, flags, out, bd,
                                  nullptr, 0, stream, nullptr, nullptr);
  if (compare_layout(n, v, k, flags).total > LCMP_NOALLOC_SCRATCH_BYTES) return LCMP_EWORKSPACE;
  void *ws = scratch_of_current_device();
  if (!ws) return LCMP_EHIP;
  return compare_impl(base, tb, ld_base, cand, tc, ld_cand, n, v, k, flags, out, bd, ws,
                      LCMP_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr);
}

size_t lcmp_bitdiff_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 1 || cols > kMaxCols || rows > kMaxRows) return 0;
  if (rows == 0) return kAlign;
  const Chunking ch = choose_chunks(rows, cols);
  return align_up((size_t)rows * (size_t)ch.nchunks * sizeof(ChunkBits));
}

static int bitdiff_impl(const void *a, int ta, int64_t lda, const void *b, int tb, int64_t ldb,
                        int64_t rows, int64_t cols, lcmp_bitdiff_row *out, void *workspace,
                        size_t ws_bytes, void *stream, void *ev_before, void *ev_after) {
  if (!dtype_ok(ta) || !dtype_ok(tb)) return LCMP_EDTYPE;
  if (rows < 0) return LCMP_EINVAL;
  if (cols < 1 || cols > kMaxCols || rows > kMaxRows || lda < cols || ldb < cols)
    return LCMP_ESHAPE;
  if (rows == 0) return empty_call(ev_before, ev_after, stream);
  if (!a || !b || !out) return LCMP_EINVAL;
  const Chunking ch = choose_chunks(rows, cols);
  const size_t need = align_up((size_t)rows * (size_t)ch.nchunks * sizeof(ChunkBits));
  if (!workspace || ws_bytes < need) return LCMP_EWORKSPACE;
  if ((uintptr_t)workspace % 16 != 0) return LCMP_EINVAL;
  StreamArgs sa;
  memset(&sa, 0, sizeof sa);
  sa.a = a;
  sa.b = b;
  sa.lda = lda;
  sa.ldb = ldb;
  sa.n = rows;
  sa.v = cols;
  sa.chunk = ch.chunk;
  sa.nchunks = ch.nchunks;
  sa.kint = 2;
  sa.bits = (ChunkBits *)workspace;
  hipStream_t s = (hipStream_t)stream;
  if (launch_row_stats(sa, ta, tb, false, true, vector_ok(a, ta, lda, b, tb, ldb), s,
                       timing(ev_before, ev_after)) != hipSuccess)
    return LCMP_EHIP;
  BitsFinalArgs fa;
  fa.bits = sa.bits;
  fa.rows = rows;
  fa.cols = cols;
  fa.nchunks = ch.nchunks;
  fa.out = (BitdiffRow *)out;
  if (launch_bitdiff_final(fa, s) != hipSuccess) return LCMP_EHIP;
  return LCMP_OK;
}

int lcmp_bitdiff(const void *a, int ta, int64_t lda, const void *b, int tb, int64_t ldb,
                 int64_t rows, int64_t cols, lcmp_bitdiff_row *out, void *workspace,
                 size_t ws_bytes, void *stream) {
  return bitdiff_impl(a, ta, lda, b, tb, ldb, rows, cols, out, workspace, ws_bytes, stream,
                      nullptr, nullptr);
}

int lcmp_bitdiff_timed(const void *a, int ta, int64_t lda, const void *b, int tb, int64_t ldb,
                       int64_t rows, int64_t cols, lcmp_bitdiff_row *out, void *workspace,
                       size_t ws_bytes, void *stream, void *ev_before, void *ev_after) {
  return bitdiff_impl(a, ta, lda, b, tb, ldb, rows, cols, out, workspace, ws_bytes, stream,
                      ev_before, ev_after);
}

int lcmp_read_probe(const void *base, int tb, int64_t ld_base, const void *cand, int tc,
                    int64_t ld_cand, int64_t n, int64_t v, void *workspace, size_t ws_bytes,
                    void *stream, void *ev_before, void *ev_after) {
  if (!dtype_ok(tb) || !dtype_ok(tc)) return LCMP_EDTYPE;
  if (n < 0) return LCMP_EINVAL;
  if (v < 2 || v > kMaxCols || n > kMaxRows || ld_base < v || ld_cand < v) return LCMP_ESHAPE;
  if (n == 0) return empty_call(ev_before, ev_after, stream);
  if (!base || !cand || !vector_ok(base, tb, ld_base, cand, tc, ld_cand)) return LCMP_EINVAL;
  const Chunking ch = choose_chunks(n, v);
  if (!workspace || ws_bytes < (size_t)n * (size_t)ch.nchunks * sizeof(uint32_t))
    return LCMP_EWORKSPACE;
  if ((uintptr_t)workspace % 16 != 0) return LCMP_EINVAL;
  StreamArgs sa;
  memset(&sa, 0, sizeof sa);
  sa.a = base;
  sa.b = cand;
  sa.lda = ld_base;
  sa.ldb = ld_cand;
  sa.n = n;
  sa.v = v;
  sa.chunk = ch.chunk;
  sa.nchunks = ch.nchunks;
  hipStream_t s = (hipStream_t)stream;
  if (launch_read_probe(sa, tb, tc, (uint32_t *)workspace, s, timing(ev_before, ev_after)) !=
      hipSuccess)
    return LCMP_EHIP;
  return LCMP_OK;
}

size_t lcmp_bin_workspace_bytes(int64_t n, int n_groups, int n_edges) {
  if (n < 0 || n > kMaxBinRows || n_groups < 1 || n_groups > kMaxGroups || n_edges < 1 || n_edges > kMaxEdges ||
      n_groups * n_edges > kMaxBins)
    return 0;
  const int rows = bin_rows_per_block(n);
  const int64_t nblk = (n + rows - 1) / rows;
  return align_up((size_t)nblk * (size_t)n_groups * n_edges * sizeof(BinAcc)) +
         align_up((size_t)nblk * (size_t)n_groups * sizeof(GroupAcc)) + kAlign;
}

int lcmp_perturb(const void *src, int ts, int64_t ld_src, void *dst, int td, int64_t ld_dst,
                 int64_t rows, int64_t cols, int mode, int param, void *stream) {
  if (!dtype_ok(ts) || !dtype_ok(td)) return LCMP_EDTYPE;
  if (rows < 0 || cols < 0) return LCMP_EINVAL;
  if (mode != LCMP_PERTURB_MANTISSA && mode != LCMP_PERTURB_E4M3 &&
      mode != LCMP_PERTURB_E4M3_SCALED)
    return LCMP_EINVAL;
  if (mode == LCMP_PERTURB_MANTISSA && (param < 0 || param > 23)) return LCMP_EINVAL;
  if (td == LCMP_BF16 &&
      !((mode == LCMP_PERTURB_MANTISSA && param <= 7) || mode == LCMP_PERTURB_E4M3))
    return LCMP_EDTYPE;  // the results would not all be bf16 values
  if (ld_src < cols || ld_dst < cols || cols > kMaxCols) return LCMP_ESHAPE;
  if (rows == 0 || cols == 0) return LCMP_OK;
  if (!src || !dst) return LCMP_EINVAL;
  PerturbArgs a;
  a.src = src;
  a.dst = dst;
  a.ld_src = ld_src;
  a.ld_dst = ld_dst;
  a.rows = rows;
  a.cols = cols;
  a.tiles = perturb_tiles(cols);
  if (rows > 0x7fffffffLL / a.tiles) return LCMP_ESHAPE;  // one block per tile
  a.ts = ts;
  a.td = td;
  a.mode = mode;
  a.param = mode == LCMP_PERTURB_MANTISSA ? param : 23;
  const size_t as = ts == LCMP_BF16 ? 8 : 16, ad = td == LCMP_BF16 ? 8 : 16;
  a.vec = (uintptr_t)src % as == 0 && ((size_t)ld_src * esize(ts)) % as == 0 &&
          (uintptr_t)dst % ad == 0 && ((size_t)ld_dst * esize(td)) % ad == 0;
  if (launch_perturb(a, (hipStream_t)stream) != hipSuccess) return LCMP_EHIP;
  return LCMP_OK;
}

int lcmp_bin_report(const double *margin, const uint8_t *flip, const double *kl_topk,
                    const double *kl_full, const uint8_t *status, const int32_t *group,
                    int n_groups, int64_t n, const double *edges, int n_edges, double big_margin,
                    lcmp_bin *bins, lcmp_group_summary *summary, void *workspace,
                    size_t ws_bytes, void *stream) {
  if (n < 0 || !bins || !summary || !edges) return LCMP_EINVAL;
  if (n > kMaxBinRows || n_groups < 1 || n_groups > kMaxGroups || n_edges < 1 ||
      n_edges > kMaxEdges || n_groups * n_edges > kMaxBins)
    return LCMP_ESHAPE;
  for (int j = 0; j < n_edges; ++j) {
    if (isnan(edges[j]) || !(edges[j] > 0.0)) return LCMP_EEDGES;
    if (j > 0 && !(edges[j] > edges[j - 1])) return LCMP_EEDGES;
  }
  if (isnan(big_margin)) return LCMP_EINVAL;
  if (n > 0 && (!margin || !flip || !kl_topk)) return LCMP_EINVAL;
  const size_t need = lcmp_bin_workspace_bytes(n, n_groups, n_edges);
  if (!workspace || ws_bytes < need) return LCMP_EWORKSPACE;
  if ((uintptr_t)workspace % 16 != 0) return LCMP_EINVAL;
  const int rows = bin_rows_per_block(n);
  const int64_t nblk = (n + rows - 1) / rows;
  BinArgs ba;
  memset(&ba, 0, sizeof ba);
  ba.margin = margin;
  ba.kl_topk = kl_topk;
  ba.kl_full = kl_full;
  ba.flip = flip;
  ba.status = status;
  ba.group = group;
  ba.n = n;
  ba.n_groups = n_groups;
  ba.n_edges = n_edges;
  for (int j = 0; j < n_edges; ++j) ba.edges[j] = edges[j];
  ba.big_margin = big_margin;
  char *ws = (char *)workspace;
  ba.part_bins = (BinAcc *)ws;
  ba.part_groups =
      (GroupAcc *)(ws + align_up((size_t)nblk * (size_t)n_groups * n_edges * sizeof(BinAcc)));
  ba.nblk = (int32_t)nblk;
  ba.rows = rows;
  ba.bins = (BinAcc *)bins;
  ba.groups = (GroupAcc *)summary;
  if (launch_bin_reduce(ba, (hipStream_t)stream) != hipSuccess) return LCMP_EHIP;
  return LCMP_OK;
}

// ---------------------------------------------------------------- compact record

size_t lcmp_record_workspace_bytes(int64_t n, int64_t v, int k_rec) {
  if (n < 0 || v < 2 || v > kMaxCols || n > kMaxRows || k_rec < 2 || k_rec > LCMP_MAX_K) return 0;
  if (n == 0) return kAlign;
  return compare_layout(n, v, k_rec, 0).total + rest_layout(n, v).bytes;
}

size_t lcmp_compare_record_workspace_bytes(int64_t n, int64_t v) {
  if (n < 0 || v < 2 || v > kMaxCols || n > kMaxRows) return 0;
  if (n == 0) return kAlign;
  return rest_layout(n, v).bytes;
}

}  // extern "C"

static int record_impl(const void *base, int tb, int64_t ld_base, int64_t n, int64_t v, int k_rec,
                       const int32_t *target, const lcmp_record *rec, void *workspace,
                       size_t ws_bytes, void *stream) {
  if (!dtype_ok(tb)) return LCMP_EDTYPE;
  if (n < 0 || !rec) return LCMP_EINVAL;
  if (v < 2 || v > kMaxCols || n > kMaxRows || k_rec < 2 || k_rec > LCMP_MAX_K || ld_base < v)
    return LCMP_ESHAPE;
  if (rec->logp_target && !target) return LCMP_EINVAL;
  if (n == 0) return LCMP_OK;
  if (!base || !record_ok(rec)) return LCMP_EINVAL;
  const CompareLayout CL = compare_layout(n, v, k_rec, 0);
  const RestLayout RL = rest_layout(n, v);
  if (!workspace || ws_bytes < CL.total + RL.bytes) return LCMP_EWORKSPACE;
  if ((uintptr_t)workspace % 16 != 0) return LCMP_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  // 1. the baseline's top-k_rec and status: the full compare of the baseline
  //    with itself, writing only those two outputs
  lcmp_row_out ro;
  memset(&ro, 0, sizeof ro);
  ro.topk_idx = rec->topk_idx;
  ro.status = rec->status;
  const int rc = compare_impl(base, tb, ld_base, base, tb, ld_base, n, v, k_rec, 0, &ro, nullptr,
                              workspace, CL.total, stream, nullptr, nullptr);
  if (rc != LCMP_OK) return rc;
  // 2. the mass outside the top-k_rec
  RestArgs ra;
  ra.x = base;
  ra.ldx = ld_base;
  ra.n = n;
  ra.v = v;
  ra.chunk = RL.ch.chunk;
  ra.nchunks = RL.ch.nchunks;
  ra.head = rec->topk_idx;
  ra.ldh = k_rec;
  ra.kh = k_rec;
  ra.out = (RestChunk *)((char *)workspace + CL.total);
  if (launch_rest_sum(ra, tb, rows_aligned(base, tb, ld_base), s) != hipSuccess) return LCMP_EHIP;
  // 3. values, rest mass and target log-probability
  RecordArgs fa;
  fa.base = base;
  fa.tb = tb;
  fa.ldb = ld_base;
  fa.n = n;
  fa.v = v;
  fa.krec = k_rec;
  fa.nchunks = RL.ch.nchunks;
  fa.rest = ra.out;
  fa.idx = rec->topk_idx;
  fa.status = rec->status;
  fa.val = rec->topk_val;
  fa.lse_rest = rec->lse_rest;
  fa.target = rec->logp_target ? target : nullptr;
  fa.logp = rec->logp_target;
  if (launch_record_final(fa, s) != hipSuccess) return LCMP_EHIP;
  return LCMP_OK;
}

static int compare_record_impl(const lcmp_record *rec, int k_rec, const void *cand, int tc,
                               int64_t ld_cand, int64_t n, int64_t v, int k,
                               const lcmp_row_out *out, void *workspace, size_t ws_bytes,
                               void *stream, void *ev_before, void *ev_after) {
  if (!dtype_ok(tc)) return LCMP_EDTYPE;
  if (n < 0 || !rec || !out) return LCMP_EINVAL;
  if (v < 2 || v > kMaxCols || n > kMaxRows || k_rec < 2 || k_rec > LCMP_MAX_K || k < 1 ||
      k > k_rec || ld_cand < v)
    return LCMP_ESHAPE;
  if (out->kl_full) return LCMP_EINVAL;  // needs the whole baseline row
  if ((out->logp_base || out->logp_cand) && !out->target) return LCMP_EINVAL;
  if (out->logp_base && !rec->logp_target) return LCMP_EINVAL;
  if (n == 0) return empty_call(ev_before, ev_after, stream);
  if (!cand || !record_ok(rec)) return LCMP_EINVAL;
  const RestLayout RL = rest_layout(n, v);
  if (!workspace || ws_bytes < RL.bytes) return LCMP_EWORKSPACE;
  if ((uintptr_t)workspace % 16 != 0) return LCMP_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  RestArgs ra;
  ra.x = cand;
  ra.ldx = ld_cand;
  ra.n = n;
  ra.v = v;
  ra.chunk = RL.ch.chunk;
  ra.nchunks = RL.ch.nchunks;
  ra.head = rec->topk_idx;
  ra.ldh = k_rec;
  ra.kh = k;
  ra.out = (RestChunk *)workspace;
  if (launch_rest_sum(ra, tc, rows_aligned(cand, tc, ld_cand), s, timing(ev_before, ev_after)) !=
      hipSuccess)
    return LCMP_EHIP;
  RecordCmpArgs ca;
  ca.idx = rec->topk_idx;
  ca.val = rec->topk_val;
  ca.lse_rest = rec->lse_rest;
  ca.rec_status = rec->status;
  ca.rec_logp = rec->logp_target;
  ca.krec = k_rec;
  ca.k = k;
  ca.nchunks = RL.ch.nchunks;
  ca.tc = tc;
  ca.cand = cand;
  ca.ldc = ld_cand;
  ca.n = n;
  ca.v = v;
  ca.rest = ra.out;
  const bool with_target = out->target && (out->logp_base || out->logp_cand);
  ca.target = with_target ? out->target : nullptr;
  ca.kl_topk = out->kl_topk;
  ca.margin = out->margin;
  ca.lse_base = out->lse_base;
  ca.lse_cand = out->lse_cand;
  ca.top1_base = out->top1_base;
  ca.top2_base = out->top2_base;
  ca.top1_cand = out->top1_cand;
  ca.flip = out->flip;
  ca.status = out->status;
  ca.topk_idx = out->topk_idx;
  ca.logp_base = with_target ? out->logp_base : nullptr;
  ca.logp_cand = with_target ? out->logp_cand : nullptr;
  if (launch_record_cmp(ca, s) != hipSuccess) return LCMP_EHIP;
  return LCMP_OK;
}

extern "C" {

int lcmp_record_baseline(const void *base, int tb, int64_t ld_base, int64_t n, int64_t v,
                         int k_rec, const int32_t *target, const lcmp_record *rec,
                         void *workspace, size_t ws_bytes, void *stream) {
  return record_impl(base, tb, ld_base, n, v, k_rec, target, rec, workspace, ws_bytes, stream);
}

int lcmp_compare_record(const lcmp_record *rec, int k_rec, const void *cand, int tc,
                        int64_t ld_cand, int64_t n, int64_t v, int k, const lcmp_row_out *out,
                        void *workspace, size_t ws_bytes, void *stream) {
  return compare_record_impl(rec, k_rec, cand, tc, ld_cand, n, v, k, out, workspace, ws_bytes,
                             stream, nullptr, nullptr);
}

int lcmp_compare_record_timed(const lcmp_record *rec, int k_rec, const void *cand, int tc,
                              int64_t ld_cand, int64_t n, int64_t v, int k,
                              const lcmp_row_out *out, void *workspace, size_t ws_bytes,
                              void *stream, void *ev_before, void *ev_after) {
  return compare_record_impl(rec, k_rec, cand, tc, ld_cand, n, v, k, out, workspace, ws_bytes,
                             stream, ev_before, ev_after);
}

}  // extern "C"
