// k_topk_kl.hip -- per-row merge of the streamed chunk records and the final
// comparison quantities, in double precision (one wave per row).
//
// With u = E/s (E = f - d = sum e*expm1(-delta)), L = lse_cand - lse_base =
// log1p(u) = ln(w/s) (w the candidate's mass), and p_i = e_i/s:
//   full KL    = sum_i p_i (delta_i + L)                 = f/s - psi(u)
//   top-k KL   = sum_S p_i phi_i + p_o psi(E_o/p_o) - psi(u)
// where psi(x) = x - log1p(x), phi_i = delta_i + expm1(-delta_i), S the
// baseline's top-k set, p_o its complement mass and E_o = u - sum_S p_i g_i
// (g_i = expm1(-delta_i)).  Both are the KL of the page "在 agent 时代如何快速验证
// kernel 对精度的影响" (section 怎么比两个分布: the KL equation and the top-20 +
// "other" bucket) rewritten so that only second-order quantities are summed:
// no difference of two nearly equal log-normalisers is ever formed.  That
// form holds while the two normalisers are close (-1/2 < u < 1).  Beyond,
// f/s and psi(u) grow with u (or E loses the candidate mass as u nears -1),
// so the first-order form is used, with L = ln(w/s) from the candidate mass:
//   full KL    = d/s + L
//   top-k KL   = sum_S p_i (delta_i + L) + p_o (ln(s_o / w_o) + L)
// with s_o and w_o the two masses outside S.  When w_o is itself a small
// difference of large sums, the same wave sums both buckets again directly
// over the row (bucket_direct).
#include "common.hpp"
#include "launch.hpp"
#include "merge.hpp"

#include <math.h>

namespace lcmp {

__device__ __forceinline__ void wave_fence2() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float load_elem(const void *p, int t, int64_t off) {
  if (t == 1) return __uint_as_float((uint32_t)((const uint16_t *)p)[off] << 16);
  return ((const float *)p)[off];
}

// The two masses outside the head set H (keff columns listed in h[], in any
// order) of one row, summed directly: per side the largest value outside H
// (log2 units: ra2, rb2), then the sum of 2^(x*kL2E - r2) in double over the
// columns outside H.  Lane l takes columns l, l + 64, ... (ascending) and
// walks the head, sorted ascending into hs[], alongside; the lanes are
// combined in a fixed order.  Whole wave; returns false when a side has no
// finite value outside H.  Rare: only rows whose one-pass bucket term is
// ill-conditioned come here, and each reads its row pair once more.
__device__ inline bool bucket_direct(const void *base, int tb, int64_t ldb, const void *cand,
                                     int tc, int64_t ldc, int64_t row, int64_t v,
                                     const int32_t *h, int keff, int32_t *hs, double &sa,
                                     double &sb, float &ra2, float &rb2) {
  const int lane = lane_id();
  // sort the head indices ascending: lane j ranks its index among the keff
  const int hj = lane < keff ? h[lane] : 0x7fffffff;
  int rank = 0;
  for (int i = 0; i < keff; ++i) rank += __shfl(hj, i, kWave) < hj ? 1 : 0;
  wave_fence2();
  if (lane < keff) hs[rank] = hj;
  wave_fence2();
  const int64_t ra = row * ldb, rb = row * ldc;
  float ma = -INFINITY, mb = -INFINITY;
  int hp = 0;
  for (int64_t c = lane; c < v; c += kWave) {
    while (hp < keff && hs[hp] < c) ++hp;
    if (hp < keff && hs[hp] == c) continue;
    ma = fmaxf(ma, load_elem(base, tb, ra + c));
    mb = fmaxf(mb, load_elem(cand, tc, rb + c));
  }
  ma = uniform(wave_max(ma));
  mb = uniform(wave_max(mb));
  if (!(ma > -INFINITY) || !(mb > -INFINITY)) return false;
  ra2 = ma * kL2E;
  rb2 = mb * kL2E;  // every term below is at most 1
  double xa = 0.0, xb = 0.0;
  hp = 0;
  for (int64_t c = lane; c < v; c += kWave) {
    while (hp < keff && hs[hp] < c) ++hp;
    if (hp < keff && hs[hp] == c) continue;
    const float x = load_elem(base, tb, ra + c), y = load_elem(cand, tc, rb + c);
    if (x > -INFINITY) xa += (double)__builtin_amdgcn_exp2f(fmaf(x, kL2E, -ra2));
    if (y > -INFINITY) xb += (double)__builtin_amdgcn_exp2f(fmaf(y, kL2E, -rb2));
  }
  sa = wave_sum(xa);
  sb = wave_sum(xb);
  return true;
}

// The row's top-k slots (C * kint of them, C <= kMaxMergeChunks) are held in
// registers, R per lane (R * 64 >= C * kint; instances for R = 1, 2, 4, 16).
constexpr int kMaxMergeChunks = 16;

template <int R>
__global__ __launch_bounds__(kWave) void k_topk_kl(FinalArgs a) {
  constexpr int kSlotRounds = R;
  __shared__ uint32_t sel_key[kMaxK];  // the kint selected slots, in slot order
  __shared__ int32_t sel_idx[kMaxK];
  __shared__ float sel_cv[kMaxK];      // the candidate logit at each selected index
  __shared__ float s_a[kMaxK];         // the same, value descending, index ascending
  __shared__ int32_t s_i[kMaxK];
  __shared__ float s_b[kMaxK];
  const int lane = lane_id();
  const int64_t row = blockIdx.x;
  const int C = a.nchunks;
  const int kint = a.kint;
  const int mcap = C * kint;            // top-k slots of the row's chunks
  const int rounds = (mcap + kWave - 1) / kWave;

  // ---- every load that does not depend on another goes out first: the chunk
  // records, the bitwise chunk records and all top-k slots (the slots past a
  // chunk's count are masked below)
  const bool has = lane < C;
  ChunkStats cs;
  if (has) cs = a.stats[row * C + lane];
  ChunkBits cb = no_bits();
  if (a.bd && has) cb = a.bits[row * C + lane];
  const int64_t tb = row * (int64_t)mcap;
  float sv[kSlotRounds];
  int sx[kSlotRounds];
#pragma unroll
  for (int q = 0; q < kSlotRounds; ++q) {
    const int e = lane + kWave * q;
    sv[q] = 0.0f;
    sx[q] = 0;
    if (q < rounds && e < mcap) {
      sv[q] = a.ta[tb + e];
      sx[q] = a.ti[tb + e];
    }
  }
  if (lane < kMaxK) {
    s_a[lane] = -INFINITY;
    s_i[lane] = -1;
    s_b[lane] = -INFINITY;
    sel_key[lane] = 0u;
    sel_idx[lane] = 0x7fffffff;
    sel_cv[lane] = -INFINITY;
  }

  // ---- the row's top-k slots as keys.  Slot e holds entry (e mod kint) of
  // chunk e / kint; empty slots get key 0, below every stored key.  Keys are
  // distinct through the index, and at least kint slots are filled (every
  // chunk stores min(kint, its length) entries).  The candidate logit at
  // every filled slot's index is fetched here, before the selection, so its
  // latency overlaps the merge; the index test only keeps a damaged record
  // from reading outside the row.
  uint32_t key[kSlotRounds];
  int idx[kSlotRounds];
  float cv[kSlotRounds];
#pragma unroll
  for (int q = 0; q < kSlotRounds; ++q) {
    key[q] = 0u;
    idx[q] = 0x7fffffff;
    cv[q] = -INFINITY;
    if (q < rounds) {
      const int e = lane + kWave * q;
      const int c = e / kint;
      // chunk c's entry count, from lane c
      const int cnt_c = __builtin_amdgcn_ds_bpermute(min(c, kWave - 1) << 2, has ? cs.cnt : 0);
      if (e < mcap && e - c * kint < cnt_c) {
        key[q] = rank_key(sv[q]);
        idx[q] = sx[q];
        if (sx[q] >= 0 && (int64_t)sx[q] < a.v) cv[q] = load_elem(a.cand, a.tc, row * a.ldc + sx[q]);
      }
    }
  }

  // the teacher-forced token's logits on both sides, also fetched early
  int tgt = -1;
  float tgt_a = NAN, tgt_b = NAN;
  if (a.target && lane == 0) {
    tgt = a.target[row];
    if (tgt >= 0 && (int64_t)tgt < a.v) {
      tgt_a = load_elem(a.base, a.tb, row * a.ldb + tgt);
      tgt_b = load_elem(a.cand, a.tc, row * a.ldc + tgt);
    }
  }

  if (a.bd) merge_bits_lanes(cb, C, a.v, a.bd + row);

  // ---- chunk sums, rescaled to the largest reference
  const double r2 = has ? cs.r2 : -INFINITY;
  const double M2 = lanes_max(r2, C);
  const int nb = lanes_sum(has ? cs.n_bad : 0, C);
  const int na = lanes_sum(has ? cs.n_ainf : 0, C);
  const int nbi = lanes_sum(has ? cs.n_binf : 0, C);
  const int nq = lanes_sum(has ? cs.n_qzero : 0, C);
  uint8_t status = 0;
  if (nb > 0)
    status = 1;  // LCMP_ROW_NONFINITE
  else if ((int64_t)na == a.v || (int64_t)nbi == a.v)
    status = 2;  // LCMP_ROW_EMPTY
  if (status) {
    if (lane == 0) {
      if (a.kl_topk) a.kl_topk[row] = NAN;
      if (a.kl_full) a.kl_full[row] = NAN;
      if (a.margin) a.margin[row] = NAN;
      if (a.lse_base) a.lse_base[row] = NAN;
      if (a.lse_cand) a.lse_cand[row] = NAN;
      if (a.top1_base) a.top1_base[row] = -1;
      if (a.top2_base) a.top2_base[row] = -1;
      if (a.top1_cand) a.top1_cand[row] = -1;
      if (a.flip) a.flip[row] = 0;
      if (a.status) a.status[row] = status;
      if (a.target) {
        if (a.logp_base) a.logp_base[row] = NAN;
        if (a.logp_cand) a.logp_cand[row] = NAN;
      }
    }
    if (a.topk_idx)
      for (int j = lane; j < a.k; j += kWave) a.topk_idx[row * a.k + j] = -1;
    return;
  }
  // a chunk without a reference held no finite logit on either side: it adds
  // nothing (it is left out rather than scaled by 0)
  const bool live = has && r2 > -INFINITY;
  const double sc = live ? exp2(r2 - M2) : 0.0;
  const double S = lanes_sum(live ? cs.s * sc : 0.0, C);
  const double D = lanes_sum(live ? cs.d * sc : 0.0, C);
  const double F = lanes_sum(live ? cs.f * sc : 0.0, C);
  const double W = lanes_sum(live ? cs.w * sc : 0.0, C);

  // ---- candidate argmax across chunks: value descending, index ascending
  const float bm = has ? cs.bmax : -INFINITY;
  const float BM = uniform(lanes_max(bm, C));
  const int bx = lanes_min((has && cs.bidx >= 0 && bm == BM) ? cs.bidx : 0x7fffffff, C);
  const int top1_cand = bx == 0x7fffffff ? -1 : bx;

  // ---- the row's top kint slots: the kint-th largest key T, two bits at a time from the top; then the ties at T
  // that are kept, lowest indices first.  The search stops as soon as exactly kint keys lie at or above its
  // prefix (those are the kint largest).  bf16 baseline values give keys whose low 16 bits are all equal
  // (zeros when positive, ones when negative), so their search ends at bit 16.
  const bool k16 = a.tb == 1;
  uint32_t T = 0;
  int nT = kWave * kSlotRounds;  // at least kint keys lie at or above T
  bool early = false;
  // each round takes the largest of the three extensions of T with at least
  // kint keys at or above it (three ballots per slot round, issued together)
#pragma unroll 1
  for (int bit = 30; bit >= (k16 ? 16 : 0); bit -= 2) {
    const uint32_t c1 = T | (1u << bit), c2 = T | (2u << bit), c3 = T | (3u << bit);
    int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
    for (int q = 0; q < kSlotRounds; ++q) {
      if (q < rounds) {
        n1 += __popcll(ballot(key[q] >= c1));
        n2 += __popcll(ballot(key[q] >= c2));
        n3 += __popcll(ballot(key[q] >= c3));
      }
    }
    if (n3 >= kint) {
      T = c3;
      nT = n3;
    } else if (n2 >= kint) {
      T = c2;
      nT = n2;
    } else if (n1 >= kint) {
      T = c1;
      nT = n1;
    }
    if (nT == kint) {
      early = true;
      break;
    }
  }
  if (k16 && !early && T < 0x80000000u) T |= 0xffffu;
  uint32_t isel = 0x7fffffffu;
  if (!early) {
    int ngt = 0, neq = 0;
#pragma unroll
    for (int q = 0; q < kSlotRounds; ++q) {
      if (q < rounds) {
        ngt += __popcll(ballot(key[q] > T));
        neq += __popcll(ballot(key[q] == T));
      }
    }
    const int need = kint - ngt;
    if (neq > need) {
      // columns are below v: the higher bits of the need-th smallest are zero
      const int cbit = a.v > 1 ? 63 - __builtin_clzll((unsigned long long)(a.v - 1)) : 0;
      uint32_t I = 0;
#pragma unroll 1
      for (int bit = cbit; bit >= 0; --bit) {
        const uint32_t c = I | (1u << bit);
        int n = 0;
#pragma unroll
        for (int q = 0; q < kSlotRounds; ++q)
          if (q < rounds) n += __popcll(ballot(key[q] == T && (uint32_t)idx[q] < c));
        if (n < need) I = c;
      }
      isel = I;
    }
  }
  // compact the kint kept slots, then order them: lane j < kint holds kept
  // entry j and counts the kept entries ahead of it
  int fill = 0;
#pragma unroll
  for (int q = 0; q < kSlotRounds; ++q) {
    if (q < rounds) {
      const bool keep = key[q] > T || (key[q] == T && (uint32_t)idx[q] <= isel);
      const uint64_t m = ballot(keep);
      const int pos = fill + prefix_count(m);
      if (keep && pos < kint) {  // exactly kint are kept when kint slots are filled
        sel_key[pos] = key[q];
        sel_idx[pos] = idx[q];
        sel_cv[pos] = cv[q];
      }
      fill += __popcll(m);
    }
  }
  wave_fence2();
  const uint32_t kj = lane < kint ? sel_key[lane] : 0u;
  const int ij = lane < kint ? sel_idx[lane] : 0x7fffffff;
  const float cj = lane < kint ? sel_cv[lane] : -INFINITY;
  int rank = 0;
  for (int i = 0; i < kint; ++i) {
    const uint32_t ki = (uint32_t)__builtin_amdgcn_readlane((int)kj, i);
    const int ii = __builtin_amdgcn_readlane(ij, i);
    rank += (ki > kj || (ki == kj && ii < ij)) ? 1 : 0;
  }
  if (lane < kint && kj != 0u) {
    s_a[rank] = rank_key_inv(kj);
    s_i[rank] = ij;
    s_b[rank] = cj;
  }
  wave_fence2();

  // ---- head terms (lanes j < k_eff)
  const int keff = (int)min((int64_t)a.k, a.v);
  const bool in_head = lane < keff;
  const float ha = in_head ? s_a[lane] : -INFINITY;
  // the candidate logit at each head index, fetched with the slots
  const float hb = in_head ? s_b[lane] : -INFINITY;
  // the normalisers' log-ratio L (uniform: every lane computes it)
  const double u = (F - D) / S;
  const bool near = u > -0.5 && u < 1.0;
  // the weights are powers of two of x * kL2E (kL2E a float, 1.3e-8 from
  // log2 e): the logarithm of a ratio of them returns to natural units
  // through 1 / (kL2E ln 2), so that a pure shift of the candidate gives
  // L = -shift exactly
  const double units = 1.0 / ((double)kL2E * kLn2);
  const double L = near ? log1p(u) : log(W / S) * units;

  const bool ainf = ha == -INFINITY, binf = hb == -INFINITY;
  double e = 0.0, eb = 0.0, tphi = 0.0, tg = 0.0, tpl = 0.0;
  int head_inf = 0;
  if (in_head && !ainf) {
    e = exp2((double)ha * (double)kL2E - M2);
    const double p = e / S;
    if (binf) {
      head_inf = 1;
      tg = -p;
    } else {
      const double dl = (double)ha - (double)hb;
      const double g = expm1(-dl);
      tphi = p * (dl + g);
      tg = p * g;
      tpl = p * (dl + L);  // p_i ln(p_i / q_i)
    }
  }
  if (in_head && !binf) eb = exp2((double)hb * (double)kL2E - M2);
  const double sum_e = wave_sum(e), sum_pphi = wave_sum(tphi), sum_pg = wave_sum(tg);
  const double sum_eb = wave_sum(eb), sum_pl = wave_sum(tpl);
  const int n_sa = __popcll(ballot(in_head && ainf));
  const int n_sb = __popcll(ballot(in_head && binf));
  const int any_head_inf = ballot(head_inf != 0) != 0;

  if (a.topk_idx)
    for (int j = lane; j < a.k; j += kWave) a.topk_idx[row * a.k + j] = j < keff ? s_i[j] : -1;

  // the top-k KL with its bucket term (uniform: every lane computes it)
  const double kl_full = nq > 0 ? INFINITY : near ? F / S - psi(u) : D / S + L;
  double klk;
  bool ill = false;  // the bucket term must be summed directly
  if (any_head_inf) {
    klk = INFINITY;
  } else {
    klk = near ? sum_pphi - psi(u) : sum_pl;
    const int64_t n_other = a.v - keff;
    const int64_t o_fin_a = n_other - ((int64_t)na - n_sa);
    const int64_t o_fin_b = n_other - ((int64_t)nbi - n_sb);
    if (o_fin_a > 0) {
      if (o_fin_b == 0) {
        klk = INFINITY;
      } else {
        const double s_o = S - sum_e;
        const double p_o = fmax(0.0, s_o / S);
        if (p_o > 0.0) {
          // The bucket term needs the candidate's mass outside S, here a
          // difference of the one-pass sums.  When that difference is small
          // against its terms it is ill-conditioned: with the normalisers
          // close, when the candidate keeps all but 2^-10 of the baseline's
          // bucket share inside S (its float-accumulated parts then dominate
          // the error); with them far apart, when the candidate's mass
          // outside S is below 2^-30 of its total (a large head weight swamps
          // it in double).  Such rows sum both buckets again directly.
          if (near) {
            double x = (u - sum_pg) / p_o;
            ill = !(x > -1.0 + 0x1p-10);
            if (!(x > -1.0)) x = -1.0 + 0x1p-52;
            klk += p_o * psi(x);
          } else {
            ill = !(W - sum_eb > W * 0x1p-30);
            const double w_o = fmax(W - sum_eb, W * 0x1p-52);
            klk += p_o * (log(s_o / w_o) * units + L);
          }
        }
      }
    }
  }
  if (ill && a.kl_topk) {
    // KL_k = sum_S p_i (delta_i + L) + p_o (ln(s_o / w_o) + L), with s_o and
    // w_o summed over the row outside S (s_i holds S; sel_idx is free now)
    double Sa, Sb;
    float Ma, Mb;
    if (bucket_direct(a.base, a.tb, a.ldb, a.cand, a.tc, a.ldc, row, a.v, s_i, keff, sel_idx,
                      Sa, Sb, Ma, Mb)) {
      const double po = Sa * exp2((double)Ma - M2) / S;
      const double lr = log(Sa) - log(Sb) + ((double)Ma - (double)Mb) * kLn2;
      klk = sum_pl + po * (lr * units + L);
    }
  }
  if (lane == 0) {
    const double lse_b = M2 * kLn2 + log(S);
    if (a.kl_topk) a.kl_topk[row] = klk;
    if (a.kl_full) a.kl_full[row] = kl_full;
    if (a.margin) a.margin[row] = (double)s_a[0] - (double)s_a[1];
    if (a.lse_base) a.lse_base[row] = lse_b;
    if (a.lse_cand) a.lse_cand[row] = lse_b + L;
    if (a.top1_base) a.top1_base[row] = s_i[0];
    if (a.top2_base) a.top2_base[row] = s_i[1];
    if (a.top1_cand) a.top1_cand[row] = top1_cand;
    if (a.flip) a.flip[row] = (uint8_t)(top1_cand != s_i[0]);
    if (a.status) a.status[row] = 0;
    if (a.target) {
      // log-probability of the teacher-forced next token on each side
      double lpb = NAN, lpc = NAN;
      if (tgt >= 0 && (int64_t)tgt < a.v) {
        lpb = (double)tgt_a - lse_b;
        lpc = (double)tgt_b - (lse_b + L);
      }
      if (a.logp_base) a.logp_base[row] = lpb;
      if (a.logp_cand) a.logp_cand[row] = lpc;
    }
  }
}

hipError_t launch_topk_kl(const FinalArgs &a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  if (a.nchunks > kMaxMergeChunks) return hipErrorInvalidValue;
  const int rounds = (a.nchunks * a.kint + kWave - 1) / kWave;
  const dim3 grid((unsigned)a.n);
  if (rounds <= 1)
    hipLaunchKernelGGL((k_topk_kl<1>), grid, dim3(kWave), 0, stream, a);
  else if (rounds <= 2)
    hipLaunchKernelGGL((k_topk_kl<2>), grid, dim3(kWave), 0, stream, a);
  else if (rounds <= 4)
    hipLaunchKernelGGL((k_topk_kl<4>), grid, dim3(kWave), 0, stream, a);
  else
    hipLaunchKernelGGL((k_topk_kl<16>), grid, dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- bitwise-only rows

__global__ __launch_bounds__(kWave) void k_bitdiff_final(BitsFinalArgs a) {
  const int64_t row = blockIdx.x;
  merge_bits(a.bits + row * a.nchunks, a.nchunks, a.cols, a.out + row);
}

hipError_t launch_bitdiff_final(const BitsFinalArgs &a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_bitdiff_final, dim3((unsigned)a.rows), dim3(kWave), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lcmp
