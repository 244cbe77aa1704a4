// merge.hpp -- per-row merge of the bitwise chunk records (device, inline).
#pragma once

#include "common.hpp"

namespace lcmp {

// Empty chunk record (the lanes past the row's chunks hold it).
__device__ __forceinline__ ChunkBits no_bits() {
  ChunkBits c;
  c.ndiff = 0;
  c.first = -1;
  c.nfa = c.nfb = 0;
  c.max_ulp = 0;
  c.pad_ = 0;
  c.max_abs = 0.0;
  c.sum_abs = c.ssd = c.ssb = 0.0;
  return c;
}

// Combine the chunk records of one row into the public record.  The whole wave
// calls it; lane c holds chunk c's record in `c` (1 <= nchunks <= 64; lanes at
// or past nchunks are ignored).  Sums run over the chunk lanes in a fixed
// order, so the result is the same on every run.
__device__ __forceinline__ void merge_bits_lanes(const ChunkBits &c, int nchunks, int64_t cols,
                                                 BitdiffRow *out) {
  const int64_t ndiff = lanes_sum(c.ndiff, nchunks);
  const int64_t first = lanes_min(c.first >= 0 ? c.first : INT64_MAX, nchunks);
  const int64_t nfa = lanes_sum(c.nfa, nchunks), nfb = lanes_sum(c.nfb, nchunks);
  const uint32_t mu = lanes_max(c.max_ulp, nchunks);
  const double ma = lanes_max(c.max_abs, nchunks);
  const double sab = lanes_sum(c.sum_abs, nchunks), ssd = lanes_sum(c.ssd, nchunks),
               ssb = lanes_sum(c.ssb, nchunks);
  if (lane_id() == 0) {
    BitdiffRow r;
    r.ndiff = ndiff;
    r.first_diff = first == INT64_MAX ? -1 : first;
    r.nonfinite_a = nfa;
    r.nonfinite_b = nfb;
    r.max_ulp = mu;
    r.pad_ = 0;
    r.max_abs = ma;
    r.sum_abs = sab;
    r.sum_sq_diff = ssd;
    r.sum_sq_base = ssb;
    r.mean_abs = sab / (double)cols;
    r.rel_l2 = ssb > 0.0 ? sqrt(ssd / ssb) : (ssd > 0.0 ? INFINITY : 0.0);
    *out = r;
  }
}

// The same, reading chunk c's record from cb[c] on lane c.
__device__ __forceinline__ void merge_bits(const ChunkBits *cb, int nchunks, int64_t cols,
                                           BitdiffRow *out) {
  const int lane = lane_id();
  const ChunkBits c = lane < nchunks ? cb[lane] : no_bits();
  merge_bits_lanes(c, nchunks, cols, out);
}

}  // namespace lcmp
