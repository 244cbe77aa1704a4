// merge.hpp -- per-row merge of the bitwise chunk records (device, inline).
#pragma once

#include "common.hpp"

namespace lcmp {

// Combine the chunk records of one row into the public record.  The whole wave
// calls it; lane c reads chunk c (nchunks <= 64).  Sums use the fixed-order
// wave reduction, so the result is the same on every run.
__device__ __forceinline__ void merge_bits(const ChunkBits *cb, int nchunks, int64_t cols,
                                           BitdiffRow *out) {
  const int lane = lane_id();
  const bool has = lane < nchunks;
  ChunkBits c;
  if (has) {
    c = cb[lane];
  } else {
    c.ndiff = 0;
    c.first = -1;
    c.nfa = c.nfb = 0;
    c.max_ulp = 0;
    c.max_abs = 0.0;
    c.sum_abs = c.ssd = c.ssb = 0.0;
  }
  const int64_t ndiff = wave_sum(c.ndiff);
  const int64_t first = wave_min(c.first >= 0 ? c.first : INT64_MAX);
  const int64_t nfa = wave_sum(c.nfa), nfb = wave_sum(c.nfb);
  const uint32_t mu = wave_max(c.max_ulp);
  const double ma = wave_max(c.max_abs);
  const double sab = wave_sum(c.sum_abs), ssd = wave_sum(c.ssd), ssb = wave_sum(c.ssb);
  if (lane == 0) {
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

}  // namespace lcmp
