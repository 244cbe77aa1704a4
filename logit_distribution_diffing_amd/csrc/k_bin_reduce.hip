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
// Reports of at most 16 blocks, 64 bins and 16 groups run both levels in one
// launch of one block (k_bin_small), with the same per-block code.
#include "common.hpp"
#include "launch.hpp"

#include <math.h>

namespace lcmp {

// LDS accumulators of one level-1 block (one wave), for up to NB bins and NG
// groups.
template <int NB, int NG>
struct BlockAcc {
  double kt[NB], kf[NB], mx[NB];
  unsigned long long cnt[NB][4];
  unsigned long long grp[NG][3];

  __device__ BinAcc bin(int t) const {
    BinAcc o;
    o.count = (int64_t)cnt[t][0];
    o.flips = (int64_t)cnt[t][1];
    o.ties = (int64_t)cnt[t][2];
    o.tie_flips = (int64_t)cnt[t][3];
    o.sum_kl_topk = kt[t];
    o.sum_kl_full = kf[t];
    o.max_kl_topk = mx[t];
    return o;
  }
  __device__ GroupAcc group(int g) const {
    GroupAcc o;
    o.big_margin_flips = (int64_t)grp[g][0];
    o.excluded = (int64_t)grp[g][1];
    o.unbinned = (int64_t)grp[g][2];
    return o;
  }
};

// Level 1 for block `blk`: its rows in batches of 64 into the accumulators.
// One wave, all 64 lanes.
template <int NB, int NG>
__device__ __forceinline__ void bin_block(const BinArgs &a, int64_t blk, BlockAcc<NB, NG> &acc) {
  const int lane = lane_id();
  const int nbins = a.n_groups * a.n_edges;
  for (int t = lane; t < nbins; t += kWave) {
    acc.kt[t] = 0.0;
    acc.kf[t] = 0.0;
    acc.mx[t] = -INFINITY;
    acc.cnt[t][0] = acc.cnt[t][1] = acc.cnt[t][2] = acc.cnt[t][3] = 0ull;
  }
  for (int g = lane; g < a.n_groups; g += kWave) acc.grp[g][0] = acc.grp[g][1] = acc.grp[g][2] = 0ull;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();

  const int64_t r0 = blk * a.rows;
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
          atomicAdd(&acc.grp[g][1], 1ull);
        } else {
          const double m = a.margin[r];
          fl = a.flip[r] != 0;
          if (fl && m > a.big_margin) atomicAdd(&acc.grp[g][0], 1ull);
          int j = 0;
          while (j < a.n_edges && !(m < a.edges[j])) ++j;
          if (j == a.n_edges) {
            atomicAdd(&acc.grp[g][2], 1ull);
          } else {
            bin = g * a.n_edges + j;
            kt = a.kl_topk[r];
            kf = a.kl_full ? a.kl_full[r] : NAN;
            tie = (m == 0.0);
            atomicAdd(&acc.cnt[bin][0], 1ull);
            if (fl) atomicAdd(&acc.cnt[bin][1], 1ull);
            if (tie) atomicAdd(&acc.cnt[bin][2], 1ull);
            if (tie && fl) atomicAdd(&acc.cnt[bin][3], 1ull);
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
        acc.kt[b] += skt;
        acc.kf[b] += skf;
        acc.mx[b] = fmax(acc.mx[b], mx);
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// The block's partials to the workspace.
template <int NB, int NG>
__device__ __forceinline__ void bin_block_store(const BinArgs &a, int64_t blk,
                                                const BlockAcc<NB, NG> &acc) {
  const int lane = lane_id();
  const int nbins = a.n_groups * a.n_edges;
  BinAcc *pb = a.part_bins + blk * nbins;
  for (int t = lane; t < nbins; t += kWave) pb[t] = acc.bin(t);
  GroupAcc *pg = a.part_groups + blk * a.n_groups;
  for (int g = lane; g < a.n_groups; g += kWave) pg[g] = acc.group(g);
}

// Level 2 for output t: bin t (t < nbins) or group t - nbins.  Lane l adds
// partials l, l+64, ... in order, then the fixed-order wave reduction
// combines the lanes.  One wave, all 64 lanes.  part(b) gives block b's
// partials: .bin(t) and .group(g).
template <class Part>
__device__ __forceinline__ void bin_final(const BinArgs &a, int t, const Part &part) {
  const int lane = lane_id();
  const int nbins = a.n_groups * a.n_edges;
  if (t < nbins) {
    int64_t c0 = 0, c1 = 0, c2 = 0, c3 = 0;
    double s0 = 0.0, s1 = 0.0, mx = -INFINITY;
    for (int b = lane; b < a.nblk; b += kWave) {
      const BinAcc p = part(b).bin(t);
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
      const GroupAcc p = part(b).group(g);
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

// The partials of block b, read back from the workspace.
struct StoredPart {
  const BinArgs &a;
  struct Ref {
    const BinArgs &a;
    int64_t b;
    __device__ BinAcc bin(int t) const { return a.part_bins[b * a.n_groups * a.n_edges + t]; }
    __device__ GroupAcc group(int g) const { return a.part_groups[b * a.n_groups + g]; }
  };
  __device__ Ref operator()(int b) const { return Ref{a, b}; }
};

__global__ __launch_bounds__(kWave) void k_bin_partial(BinArgs a) {
  __shared__ BlockAcc<kMaxBins, kMaxGroups> acc;
  bin_block(a, blockIdx.x, acc);
  bin_block_store(a, blockIdx.x, acc);
}

// One wave per bin (then per group).
__global__ __launch_bounds__(kWave) void k_bin_final(BinArgs a) {
  bin_final(a, blockIdx.x, StoredPart{a});
}

// Small reports in one launch: wave w is level-1 block w, with its own LDS
// accumulators; after the block barrier the waves take the level-2 outputs in
// turn and read the partials from LDS.  The same per-block and per-output
// code, and the same values, as the two kernels above: the same bits.
constexpr int kSmallWaves = 16;
constexpr int kSmallBins = 64, kSmallGroups = 16, kSmallBlocks = kSmallWaves;
__global__ __launch_bounds__(kSmallWaves * kWave) void k_bin_small(BinArgs a) {
  using Acc = BlockAcc<kSmallBins, kSmallGroups>;
  __shared__ Acc acc[kSmallWaves];
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  if (w < a.nblk) bin_block(a, w, acc[w]);
  __syncthreads();
  const int nout = a.n_groups * a.n_edges + a.n_groups;
  for (int t = w; t < nout; t += kSmallWaves)
    bin_final(a, t, [&](int b) -> const Acc & { return acc[b]; });
}

hipError_t launch_bin_reduce(const BinArgs &a, hipStream_t stream) {
  if (a.nblk <= kSmallBlocks && a.n_groups * a.n_edges <= kSmallBins &&
      a.n_groups <= kSmallGroups) {
    hipLaunchKernelGGL(k_bin_small, dim3(1), dim3(kSmallWaves * kWave), 0, stream, a);
    return hipGetLastError();
  }
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
