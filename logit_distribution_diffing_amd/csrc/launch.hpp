// launch.hpp -- argument records and host-side launchers shared by the
// translation units of liblcmp (internal; not part of the C ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace lcmp {

// streaming pass (k_row_stats): one wave per (row, chunk)
struct StreamArgs {
  const void *a, *b;
  int64_t lda, ldb;  // elements
  int64_t n, v;      // rows, columns used
  int64_t chunk;     // chunk length in elements, a multiple of kSpan
  int32_t nchunks;   // chunks per row
  int32_t kint;      // top-k entries kept per chunk
  ChunkStats *stats;  // [n * nchunks]  (compare)
  ChunkBits *bits;    // [n * nchunks]  (bitwise)
  float *ta;          // [n * nchunks * kint] top-k candidate values and indices
  int32_t *ti;
};

// per-row merge and finalize (k_topk_kl)
struct FinalArgs {
  const ChunkStats *stats;
  const ChunkBits *bits;  // NULL: no bitwise output
  const float *ta;
  const int32_t *ti;
  const void *cand;  // candidate logits, read at the top-k indices
  int32_t tc;
  int64_t ldc;
  const void *base;  // baseline logits, read at the target index
  int32_t tb;
  int64_t ldb;
  const int32_t *target;  // NULL: no target log-probabilities
  double *logp_base, *logp_cand;
  int64_t n, v;
  int32_t nchunks, kint, k;
  double *kl_topk, *kl_full, *margin, *lse_base, *lse_cand;
  int32_t *top1_base, *top2_base, *top1_cand;
  uint8_t *flip, *status;
  int32_t *topk_idx;
  BitdiffRow *bd;
};

// per-row merge of bitwise chunks (k_bitdiff)
struct BitsFinalArgs {
  const ChunkBits *bits;
  int64_t rows, cols;
  int32_t nchunks;
  BitdiffRow *out;
};

// one margin bin of one group, plus per-group counters (k_bin_reduce)
struct BinAcc {
  int64_t count, flips, ties, tie_flips;
  double sum_kl_topk, sum_kl_full, max_kl_topk;
};
struct GroupAcc {
  int64_t big_margin_flips, excluded, unbinned;
};

// Largest row count of a bin report (level-1 block count stays in 32 bits).
constexpr int64_t kMaxBinRows = (int64_t)1 << 36;  // LCMP_MAX_BIN_ROWS

// Rows of one level-1 block (one wave): 64-row blocks spread a report over
// many CUs; for long reports the block grows so that there are at most 4096
// blocks (their partials stay a small fraction of the rows read).
__host__ __device__ inline int bin_rows_per_block(int64_t n) {
  int64_t r = 64;
  while ((n + r - 1) / r > 4096 && r < ((int64_t)1 << 24)) r *= 2;
  return (int)r;
}
constexpr int kMaxBins = 256;           // n_groups * n_edges
constexpr int kMaxGroups = 256;
constexpr int kMaxEdges = 32;

struct BinArgs {
  const double *margin, *kl_topk, *kl_full;
  const uint8_t *flip, *status;
  const int32_t *group;
  int64_t n;
  int32_t n_groups, n_edges;
  double edges[kMaxEdges];
  double big_margin;
  BinAcc *part_bins;      // [nblk * n_groups * n_edges]
  GroupAcc *part_groups;  // [nblk * n_groups]
  int32_t nblk;
  int32_t rows;           // rows per level-1 block
  BinAcc *bins;           // [n_groups * n_edges]
  GroupAcc *groups;       // [n_groups]
};

// precision perturbation (k_perturb.hip)
struct PerturbArgs {
  const void *src;
  void *dst;
  int64_t ld_src, ld_dst, rows, cols, tiles;
  int32_t ts, td, mode, param;
  bool vec;  // rows of both sides aligned for 4-element vector accesses
};
int64_t perturb_tiles(int64_t cols);

// ---- compact baseline record
// One per (row, chunk) of the one-side pass: s = sum of 2^((y - r) * log2e)
// over the chunk's columns outside the head set, r the reference (-FLT_MAX
// before any finite value), and the chunk's largest value over all columns
// with its lowest column (-1 if none).
struct RestChunk {
  double s;
  float r, bmax;
  int32_t bidx, pad_;
};
struct RestArgs {
  const void *x;
  int64_t ldx;
  int64_t n, v, chunk;  // chunk: a multiple of kRestChunkQuantum columns
  int32_t nchunks;
  const int32_t *head;  // [n, ldh]: the first kh entries are excluded (-1 = none)
  int64_t ldh;
  int32_t kh;
  RestChunk *out;  // [n * nchunks]
};
constexpr int kRestChunkQuantum = 1024;

// Build the record from the full-compare outputs of the baseline against itself
// (head indices and status already in place) and the rest sums.
struct RecordArgs {
  const void *base;
  int32_t tb;
  int64_t ldb, n, v;
  int32_t krec, nchunks;
  const RestChunk *rest;
  const int32_t *idx;    // [n, krec]
  const uint8_t *status;
  float *val;            // [n, krec]
  double *lse_rest;
  const int32_t *target;  // NULL: no target log-probability
  double *logp;
};

// Compare a candidate against a record.
struct RecordCmpArgs {
  const int32_t *idx;
  const float *val;
  const double *lse_rest;
  const uint8_t *rec_status;
  const double *rec_logp;
  int32_t krec, k, nchunks, tc;
  const void *cand;
  int64_t ldc, n, v;
  const RestChunk *rest;
  const int32_t *target;
  double *kl_topk, *margin, *lse_base, *lse_cand;
  int32_t *top1_base, *top2_base, *top1_cand;
  uint8_t *flip, *status;
  int32_t *topk_idx;
  double *logp_base, *logp_cand;
};
// Optional timing of a streaming kernel: events given to the kernel's own
// dispatch (hipExtLaunchKernelGGL), so they take its start and end time and no
// marker is added to the stream.  With nothing to launch both are recorded
// back to back.
struct Timing {
  hipEvent_t before = nullptr, after = nullptr;
};
hipError_t record_empty(const Timing &t, hipStream_t stream);

hipError_t launch_rest_sum(const RestArgs &a, int tx, bool vec, hipStream_t stream,
                           const Timing &t = Timing());
hipError_t launch_record_final(const RecordArgs &a, hipStream_t stream);
hipError_t launch_record_cmp(const RecordCmpArgs &a, hipStream_t stream);
hipError_t launch_perturb(const PerturbArgs &a, hipStream_t stream);

hipError_t launch_row_stats(const StreamArgs &a, int ta, int tb, bool cmp, bool bits, bool vec,
                            hipStream_t stream, const Timing &t = Timing());
hipError_t launch_topk_kl(const FinalArgs &a, hipStream_t stream);
hipError_t launch_bitdiff_final(const BitsFinalArgs &a, hipStream_t stream);
hipError_t launch_bin_reduce(const BinArgs &a, hipStream_t stream);
hipError_t launch_read_probe(const StreamArgs &a, int ta, int tb, uint32_t *sink,
                             hipStream_t stream, const Timing &t = Timing());

}  // namespace lcmp
