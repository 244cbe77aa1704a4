// k_bin_reduce.hip -- flip counts and KL sums per margin bin and group
// (page "在 agent 时代如何快速验证 kernel 对精度的影响", section 三者联合起来验证精度问题:
// flips are judged per margin bin, and a flip at a large margin is a stop).
//
// Two levels with a fixed order, so repeated calls are bit-identical:
//   level 1: one wave per block of 64 rows (more for reports over 262144 rows);
//            each 64-row batch is split by bin, every bin's values are
//            summed with a fixed-order wave reduction and added to the block's LDS
//            accumulator in batch order; integer counts go through LDS
//            atomics (exact, order-free).
//   level 2: one wave per bin (and per group) adds the block partials in a
//            fixed lane-then-wave-reduction order.
#include "common.hpp"
#include "launch.hpp"

#include <math.h>

namespace lcmp {

__global__ __launch_bounds__(kWave) void k_bin_partial(BinArgs a) {
  __shared__ double acc_kt[kMaxBins], acc_kf[kMaxBins], acc_mx[kMaxBins];
  __shared__ unsigned long long cnt[kMaxBins][4];
  __shared__ unsigned long long grp[kMaxGroups][3];
  const int lane = lane_id();
  const int nbins = a.n_groups * a.n_edges;
  for (int t = lane; t < nbins; t += kWave) {
    acc_kt[t] = 0.0;
    acc_kf[t] = 0.0;
    acc_mx[t] = -INFINITY;
    cnt[t][0] = cnt[t][1] = cnt[t][2] = cnt[t][3] = 0ull;
  }
  for (int g = lane; g < a.n_groups; g += kWave) grp[g][0] = grp[g][1] = grp[g][2] = 0ull;
  __syncthreads();

  const int64_t r0 = (int64_t)blockIdx.x * a.rows;
  const int64_t r1 = min(a.n, r0 + a.rows);
  for (int64_t base = r0; base < r1; base += kWave) {
    const int64_t r = base + lane;
    int bin = -1;  // flat bin id, or -1 when this lane adds to no bin
    double kt = 0.0, kf = 0.0;
    bool fl = false, tie = false;
    if (r < r1) {
      const int g = a.group ? a.group[r] : 0;
      if (g >= 0 && g < a.n_groups) {
        if (a.status && a.status[r] != 0) {
          atomicAdd(&grp[g][1], 1ull);
        } else {
          const double m = a.margin[r];
          fl = a.flip[r] != 0;
          if (fl && m > a.big_margin) atomicAdd(&grp[g][0], 1ull);
          int j = 0;
          while (j < a.n_edges && !(m < a.edges[j])) ++j;
          if (j == a.n_edges) {
            atomicAdd(&grp[g][2], 1ull);
          } else {
            bin = g * a.n_edges + j;
            kt = a.kl_topk[r];
            kf = a.kl_full ? a.kl_full[r] : NAN;
            tie = (m == 0.0);
            atomicAdd(&cnt[bin][0], 1ull);
            if (fl) atomicAdd(&cnt[bin][1], 1ull);
            if (tie) atomicAdd(&cnt[bin][2], 1ull);
            if (tie && fl) atomicAdd(&cnt[bin][3], 1ull);
          }
        }
      }
    }
    // floating sums: one bin at a time, lowest pending lane's bin first
    uint64_t pending = ballot(bin >= 0);
    while (pending) {
      const int leader = __builtin_ctzll(pending);
      const int b = __builtin_amdgcn_readlane(bin, leader);
      const bool mine = (bin == b);
      pending &= ~ballot(mine);
      const double skt = wave_sum(mine ? kt : 0.0);
      const double skf = wave_sum(mine ? kf : 0.0);
      const double mx = wave_max(mine ? kt : -INFINITY);
      if (lane == 0) {
        acc_kt[b] += skt;
        acc_kf[b] += skf;
        acc_mx[b] = fmax(acc_mx[b], mx);
      }
    }
  }
  __syncthreads();
  BinAcc *pb = a.part_bins + (int64_t)blockIdx.x * nbins;
  for (int t = lane; t < nbins; t += kWave) {
    BinAcc o;
    o.count = (int64_t)cnt[t][0];
    o.flips = (int64_t)cnt[t][1];
    o.ties = (int64_t)cnt[t][2];
    o.tie_flips = (int64_t)cnt[t][3];
    o.sum_kl_topk = acc_kt[t];
    o.sum_kl_full = acc_kf[t];
    o.max_kl_topk = acc_mx[t];
    pb[t] = o;
  }
  GroupAcc *pg = a.part_groups + (int64_t)blockIdx.x * a.n_groups;
  for (int g = lane; g < a.n_groups; g += kWave) {
    GroupAcc o;
    o.big_margin_flips = (int64_t)grp[g][0];
    o.excluded = (int64_t)grp[g][1];
    o.unbinned = (int64_t)grp[g][2];
    pg[g] = o;
  }
}

// One wave per bin (then per group): lane l adds partials l, l+64, ... in order,
// then the fixed-order wave reduction combines the lanes.
__global__ __launch_bounds__(kWave) void k_bin_final(BinArgs a) {
  const int lane = lane_id();
  const int nbins = a.n_groups * a.n_edges;
  const int t = blockIdx.x;
  if (t < nbins) {
    int64_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;
    double s0 = 0.0, s1 = 0.0, mx = -INFINITY;
    for (int b = lane; b < a.nblk; b += kWave) {
      const BinAcc p = a.part_bins[(int64_t)b * nbins + t];
      c0 += p.count;
      c1 += p.flips;
      c2 += p.ties;
      c3 += p.tie_flips;
      s0 += p.sum_kl_topk;
      s1 += p.sum_kl_full;
      mx = fmax(mx, p.max_kl_topk);
    }
    BinAcc o;
    o.count = wave_sum(c0);
    o.flips = wave_sum(c1);
    o.ties = wave_sum(c2);
    o.tie_flips = wave_sum(c3);
    o.sum_kl_topk = wave_sum(s0);
    o.sum_kl_full = wave_sum(s1);
    o.max_kl_topk = wave_max(mx);
    if (lane == 0) a.bins[t] = o;
  } else {
    const int g = t - nbins;
    int64_t c0 = 0, c1 = 0, c2 = 0;
    for (int b = lane; b < a.nblk; b += kWave) {
      const GroupAcc p = a.part_groups[(int64_t)b * a.n_groups + g];
      c0 += p.big_margin_flips;
      c1 += p.excluded;
      c2 += p.unbinned;
    }
    GroupAcc o;
    o.big_margin_flips = wave_sum(c0);
    o.excluded = wave_sum(c1);
    o.unbinned = wave_sum(c2);
    if (lane == 0) a.groups[g] = o;
  }
}

hipError_t launch_bin_reduce(const BinArgs &a, hipStream_t stream) {
  if (a.nblk > 0) {
    hipLaunchKernelGGL(k_bin_partial, dim3((unsigned)a.nblk), dim3(kWave), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_bin_final, dim3((unsigned)(a.n_groups * a.n_edges + a.n_groups)),
                     dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lcmp
