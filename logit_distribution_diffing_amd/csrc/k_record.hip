// k_record.hip -- per-row kernels of the compact baseline record (one wave
// per row, double precision).
//
// The ground truth is recorded once and every candidate is compared against
// that record (page "在 agent 时代如何快速验证 kernel 对精度的影响", section 先要有一个
// ground truth).  A record row keeps the baseline's k_rec largest logits
// (value descending, index ascending), ln of the mass outside them, and the
// row status; that is all the top-k + "other" comparison (section 怎么比两个分布)
// needs of the baseline.  Comparing with the first k <= k_rec entries:
//   R  = ln(exp(lse_rest) + sum_{k <= j < k_rec} exp(val_j))   baseline bucket
//   L  = ln(exp(R) + sum_{j < k} exp(val_j))                    baseline normaliser
//   Ry = ln of the candidate's mass outside the head (the one-side pass)
//   Lc = ln(exp(Ry) + sum_{j < k} exp(y[idx_j]))                candidate normaliser
//   KL = sum_{j < k} p_j (ln p_j - ln q_j) + p_o (ln p_o - ln q_o)
// with ln p_j = val_j - L, ln q_j = y[idx_j] - Lc, ln p_o = R - L, ln q_o = Ry - Lc.
// Every normaliser is built from the same terms as the probabilities it
// divides, so the rounding of the streamed sums enters the KL only multiplied
// by the difference of the two bucket masses.
#include "common.hpp"
#include "launch.hpp"

#include <math.h>

namespace lcmp {

namespace {

__device__ __forceinline__ double load_value(const void *p, int t, int64_t ld, int64_t row,
                                             int64_t col) {
  const int64_t o = row * ld + col;
  if (t == 1) return (double)__uint_as_float((uint32_t)((const uint16_t *)p)[o] << 16);
  return (double)((const float *)p)[o];
}

// ln(exp(extra) + sum over lanes of exp(x)) with -inf terms adding nothing
__device__ __forceinline__ double log_add_lanes(double x, double extra) {
  const double m = wave_max(fmax(x, extra));
  if (m == -INFINITY) return -INFINITY;
  const double s = wave_sum(x > -INFINITY ? exp(x - m) : 0.0);
  return m + log(s + (extra > -INFINITY ? exp(extra - m) : 0.0));
}

// Merge of one row's chunk records from the one-side pass.
struct RestTotal {
  double lse;  // ln of the mass outside the head, -inf if none
  bool bad;    // a NaN, or +inf outside the head
  int bidx;    // lowest column of the row maximum, -1 if the row is all -inf
};

__device__ __forceinline__ RestTotal merge_rest(const RestChunk *rc_row, int C, int lane) {
  const bool has = lane < C;
  RestChunk rc;
  rc.s = 0.0;
  rc.r = -INFINITY;
  rc.bmax = -INFINITY;
  rc.bidx = -1;
  if (has) rc = rc_row[lane];
  const double r = has ? (double)rc.r : -INFINITY;
  const double M = wave_max(r);
  // a chunk reference of +inf makes the term NaN, which flags the row
  const double S = wave_sum(has ? rc.s * exp2((r - M) * (double)kL2E) : 0.0);
  RestTotal t;
  t.bad = !(S == S) || M == INFINITY;
  t.lse = S > 0.0 ? M + log2(S) / (double)kL2E : -INFINITY;
  const float bm = wave_max(has ? rc.bmax : -INFINITY);
  const int bi = wave_min((has && rc.bmax == bm && rc.bidx >= 0) ? rc.bidx : 0x7fffffff);
  t.bidx = bi == 0x7fffffff ? -1 : bi;
  return t;
}

__global__ __launch_bounds__(kWave) void k_record_final(RecordArgs a) {
  const int lane = lane_id();
  const int64_t row = blockIdx.x;
  const RestTotal rt = merge_rest(a.rest + row * a.nchunks, a.nchunks, lane);
  const uint8_t st = a.status[row];
  const bool in = lane < a.krec;
  const int id = in ? a.idx[row * a.krec + lane] : -1;
  if (st) {
    if (in) a.val[row * a.krec + lane] = NAN;
    if (lane == 0) {
      a.lse_rest[row] = NAN;
      if (a.logp) a.logp[row] = NAN;
    }
    return;
  }
  const double x = (id >= 0 && (int64_t)id < a.v) ? load_value(a.base, a.tb, a.ldb, row, id)
                                                   : -INFINITY;
  if (in) a.val[row * a.krec + lane] = (float)x;  // exact: x is a stored value
  if (lane == 0) a.lse_rest[row] = rt.lse;
  if (a.logp) {
    const double L = log_add_lanes(x, rt.lse);
    if (lane == 0) {
      const int t = a.target[row];
      a.logp[row] =
          (t >= 0 && (int64_t)t < a.v) ? load_value(a.base, a.tb, a.ldb, row, t) - L : NAN;
    }
  }
}

__global__ __launch_bounds__(kWave) void k_record_cmp(RecordCmpArgs a) {
  const int lane = lane_id();
  const int64_t row = blockIdx.x;
  // independent loads first: chunk records, record entries, target
  const RestTotal rt = merge_rest(a.rest + row * a.nchunks, a.nchunks, lane);
  const uint8_t rs = a.rec_status[row];
  const bool in_rec = lane < a.krec, in_head = lane < a.k;
  const int id = in_rec ? a.idx[row * a.krec + lane] : -1;
  const double x = in_rec ? (double)a.val[row * a.krec + lane] : -INFINITY;
  const bool hv = in_head && id >= 0 && (int64_t)id < a.v;
  const double y = hv ? load_value(a.cand, a.tc, a.ldc, row, id) : -INFINITY;
  const double lr = a.lse_rest[row];

  // status: the record's own, then the candidate's (NaN anywhere, +inf in the
  // stream or in the head, or an all -inf row)
  const bool head_bad = ballot(hv && (y != y || y == INFINITY)) != 0;
  uint8_t st = 0;
  if ((rs & 1u) || rt.bad || head_bad)
    st = 1;  // LCMP_ROW_NONFINITE
  else if (rs != 0 || rt.bidx < 0)
    st = 2;  // LCMP_ROW_EMPTY
  if (a.topk_idx && in_head) a.topk_idx[row * a.k + lane] = st ? -1 : id;
  if (st) {
    if (lane == 0) {
      if (a.kl_topk) a.kl_topk[row] = NAN;
      if (a.margin) a.margin[row] = NAN;
      if (a.lse_base) a.lse_base[row] = NAN;
      if (a.lse_cand) a.lse_cand[row] = NAN;
      if (a.top1_base) a.top1_base[row] = -1;
      if (a.top2_base) a.top2_base[row] = -1;
      if (a.top1_cand) a.top1_cand[row] = -1;
      if (a.flip) a.flip[row] = 0;
      if (a.status) a.status[row] = st;
      if (a.logp_base) a.logp_base[row] = NAN;
      if (a.logp_cand) a.logp_cand[row] = NAN;
    }
    return;
  }

  // baseline side from the record, candidate side from the head and the stream
  const bool ext = in_rec && !in_head && id >= 0;
  const double R = log_add_lanes(ext ? x : -INFINITY, lr);
  const double L = log_add_lanes(hv ? x : -INFINITY, R);
  const double Ry = rt.lse;
  const double Lc = log_add_lanes(hv ? y : -INFINITY, Ry);

  bool inf_k = ballot(hv && x > -INFINITY && y == -INFINITY) != 0;
  double term = 0.0;
  if (hv && x > -INFINITY && y > -INFINITY) {
    const double lp = x - L, lq = y - Lc;
    term = exp(lp) * (lp - lq);
  }
  double klk = wave_sum(term);
  if (R > -INFINITY) {
    if (Ry == -INFINITY) {
      inf_k = true;  // baseline mass in the bucket, none on the candidate side
    } else {
      const double lpo = R - L, lqo = Ry - Lc;
      klk += exp(lpo) * (lpo - lqo);
    }
  }
  const double x0 = __shfl(x, 0, kWave), x1 = __shfl(x, 1, kWave);
  const int id0 = __shfl(id, 0, kWave), id1 = __shfl(id, 1, kWave);
  if (lane == 0) {
    if (a.kl_topk) a.kl_topk[row] = inf_k ? INFINITY : klk;
    if (a.margin) a.margin[row] = x0 - x1;
    if (a.lse_base) a.lse_base[row] = L;
    if (a.lse_cand) a.lse_cand[row] = Lc;
    if (a.top1_base) a.top1_base[row] = id0;
    if (a.top2_base) a.top2_base[row] = id1;
    if (a.top1_cand) a.top1_cand[row] = rt.bidx;
    if (a.flip) a.flip[row] = (uint8_t)(rt.bidx != id0);
    if (a.status) a.status[row] = 0;
    if (a.target) {
      const int t = a.target[row];
      const bool ok = t >= 0 && (int64_t)t < a.v;
      if (a.logp_base) a.logp_base[row] = ok ? a.rec_logp[row] : NAN;
      if (a.logp_cand) a.logp_cand[row] = ok ? load_value(a.cand, a.tc, a.ldc, row, t) - Lc : NAN;
    }
  }
}

}  // namespace

hipError_t launch_record_final(const RecordArgs &a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_record_final, dim3((unsigned)a.n), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_record_cmp(const RecordCmpArgs &a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_record_cmp, dim3((unsigned)a.n), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lcmp
