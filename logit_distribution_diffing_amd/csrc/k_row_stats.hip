// k_row_stats.hip -- the streaming pass of the logit comparison (gfx950).
//
// One wave64 owns one (row, chunk) item and reads each element pair of its
// chunk exactly once from HBM.  Per element pair (a = baseline, b = candidate
// logit) it keeps, against a wave-uniform exp2 reference r2:
//   s = sum e,  d = sum e*delta,  f = sum e*phi(delta)
// with e = 2^(a*log2e - r2), delta = a - b and phi(delta) = delta + expm1(-delta).
// The finalize forms KL(P||Q) = f/s - psi(E/s), E = f - d, from these sums
// (teacher-forced full-vocabulary KL of the page "在 agent 时代如何快速验证 kernel
// 对精度的影响", section 怎么比两个分布).  Along the way it tracks the candidate
// argmax and the baseline top-k candidates (threshold filter into an LDS
// buffer, radix-select flushes), and optionally the bitwise statistics of the
// pair (differing patterns, first differing column, ULP distance, error norms;
// page "Kestrel_VLLM - 18", section 二, and page "海光 DCU 实测", sections 1 and 7).
//
// Element mapping inside one wave step of 512 elements: when either side is
// fp32, lane l takes elements [4l, 4l+4) and [256+4l, 256+4l+4), so each load
// instruction of the wave covers one contiguous run; when both sides are bf16,
// lane l takes [8l, 8l+8) with one 16-byte load per side.
#include "common.hpp"
#include "launch.hpp"

#include <math.h>

namespace lcmp {

constexpr int kFlushAt = 192;  // flush the candidate buffer once it holds this many

struct WaveState {
  // softmax sums (per lane, double across 8-element runs)
  double s, d, f;
  // uniform exp2 reference r2h + r2l: r2l is 0 unless the logits are so large
  // (|r2h| >= 2^28) that one float cannot hold the reference within a unit;
  // such chunks take the exact path throughout
  float r2h, r2l, gate;
  bool huge;
  // candidate argmax (uniform)
  float bmax;
  int bidx;
  // top-k threshold key (uniform) and buffer fill
  float tau_a;
  int tau_i, cnt;
  bool tau_set;
  // counters (per lane)
  int n_bad, n_ainf, n_binf, n_qzero;
  // bitwise statistics
  int64_t ndiff, first;  // uniform
  uint32_t max_ulp;
  float max_abs;
  double max_abs_d, sab, ssd, ssb;
  int nfa, nfb;
};

__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------- top-k buffer

// Reduce the wave's candidate buffer to exactly `kint` entries (the largest
// keys: value descending, index ascending) and raise the threshold to the
// kint-th key.  Called with the whole wave active; cnt > kint.
__device__ void flush_candidates(float *ba, float *bb, int *bi, WaveState &st, int kint) {
  wave_fence();
  const int lane = lane_id();
  const int per = (st.cnt + kWave - 1) / kWave;  // 1..4, uniform
  float va[4], vb[4];
  int ix[4];
  uint32_t key[4];
  bool ok[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + kWave * q;
    ok[q] = q < per && e < st.cnt;
    va[q] = ok[q] ? ba[e] : 0.0f;
    vb[q] = ok[q] ? bb[e] : 0.0f;
    ix[q] = ok[q] ? bi[e] : 0;
    key[q] = rank_key(va[q]);
  }
  // kint-th largest value key, one bit at a time from the top
  uint32_t T = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t c = T | (1u << bit);
    int n = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) n += __popcll(ballot(ok[q] && key[q] >= c));
    if (n >= kint) T = c;
  }
  int ngt = 0, neq = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ngt += __popcll(ballot(ok[q] && key[q] > T));
    neq += __popcll(ballot(ok[q] && key[q] == T));
  }
  const int need = kint - ngt;  // >= 1 entries taken among the ties at T
  int isel = 0x7fffffff;
  if (neq > need) {
    // need-th smallest index among the ties
    uint32_t I = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t c = I | (1u << bit);
      int n = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) n += __popcll(ballot(ok[q] && key[q] == T && (uint32_t)ix[q] < c));
      if (n < need) I = c;
    }
    isel = (int)I;
  }
  bool keep[4];
  int tie_hi = -1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    keep[q] = ok[q] && (key[q] > T || (key[q] == T && ix[q] <= isel));
    if (keep[q] && key[q] == T) tie_hi = max(tie_hi, ix[q]);
  }
  wave_fence();
  int fill = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t m = ballot(keep[q]);
    const int pos = fill + prefix_count(m);
    if (keep[q]) {
      ba[pos] = va[q];
      bb[pos] = vb[q];
      bi[pos] = ix[q];
    }
    fill += __popcll(m);
  }
  wave_fence();
  st.cnt = fill;
  st.tau_a = rank_key_inv(T);
  st.tau_i = wave_max(tie_hi);
  st.tau_set = true;
}

// ---------------------------------------------------------------- element mapping

template <bool MAPB>
__device__ __forceinline__ int lane_offset(int lane, int j) {
  if (MAPB) return 8 * lane + j;
  return (j < 4 ? 0 : 256) + 4 * lane + (j & 3);
}

template <int T>
__device__ __forceinline__ uint32_t load_pattern(const char *row, int64_t i) {
  if (T == 1) return (uint32_t)(*(const uint16_t *)(row + 2 * i)) << 16;
  return *(const uint32_t *)(row + 4 * i);
}

// Raw registers of one wave step (one lane's 8 elements of each side).
template <int TA, int TB>
struct Raw {
  static constexpr bool MAPB = (TA == 1 && TB == 1);
  u32x4 a0, a1, b0, b1;  // fp32: two 16-byte pieces; bf16 map A: .xy used; map B: a0 only
};

template <int TA, int TB>
__device__ __forceinline__ void load_vec(Raw<TA, TB> &r, const char *ra, const char *rb, int64_t base,
                                         int lane) {
  if (Raw<TA, TB>::MAPB) {
    r.a0 = __builtin_nontemporal_load((const u32x4 *)(ra + 2 * (base + 8 * lane)));
    r.b0 = __builtin_nontemporal_load((const u32x4 *)(rb + 2 * (base + 8 * lane)));
    return;
  }
  const int64_t o0 = base + 4 * lane, o1 = base + 256 + 4 * lane;
  if (TA == 0) {
    r.a0 = __builtin_nontemporal_load((const u32x4 *)(ra + 4 * o0));
    r.a1 = __builtin_nontemporal_load((const u32x4 *)(ra + 4 * o1));
  } else {
    u32x2 w0 = __builtin_nontemporal_load((const u32x2 *)(ra + 2 * o0));
    u32x2 w1 = __builtin_nontemporal_load((const u32x2 *)(ra + 2 * o1));
    r.a0 = u32x4{w0.x, w0.y, 0u, 0u};
    r.a1 = u32x4{w1.x, w1.y, 0u, 0u};
  }
  if (TB == 0) {
    r.b0 = __builtin_nontemporal_load((const u32x4 *)(rb + 4 * o0));
    r.b1 = __builtin_nontemporal_load((const u32x4 *)(rb + 4 * o1));
  } else {
    u32x2 w0 = __builtin_nontemporal_load((const u32x2 *)(rb + 2 * o0));
    u32x2 w1 = __builtin_nontemporal_load((const u32x2 *)(rb + 2 * o1));
    r.b0 = u32x4{w0.x, w0.y, 0u, 0u};
    r.b1 = u32x4{w1.x, w1.y, 0u, 0u};
  }
}

// fp32-space bit patterns of the 8 elements of one side
template <int T, bool MAPB>
__device__ __forceinline__ void decode(const u32x4 &p0, const u32x4 &p1, uint32_t (&u)[8]) {
  if (MAPB) {
    u[0] = p0.x << 16; u[1] = p0.x & 0xffff0000u;
    u[2] = p0.y << 16; u[3] = p0.y & 0xffff0000u;
    u[4] = p0.z << 16; u[5] = p0.z & 0xffff0000u;
    u[6] = p0.w << 16; u[7] = p0.w & 0xffff0000u;
  } else if (T == 0) {
    u[0] = p0.x; u[1] = p0.y; u[2] = p0.z; u[3] = p0.w;
    u[4] = p1.x; u[5] = p1.y; u[6] = p1.z; u[7] = p1.w;
  } else {
    u[0] = p0.x << 16; u[1] = p0.x & 0xffff0000u;
    u[2] = p0.y << 16; u[3] = p0.y & 0xffff0000u;
    u[4] = p1.x << 16; u[5] = p1.x & 0xffff0000u;
    u[6] = p1.y << 16; u[7] = p1.y & 0xffff0000u;
  }
}

// Bounds-checked element loads (ragged tail, unaligned rows); positions past
// `hi` read as -inf on both sides and are masked out of every statistic.
template <int TA, int TB, bool MAPB>
__device__ __forceinline__ uint32_t load_checked(uint32_t (&ua)[8], uint32_t (&ub)[8], const char *ra,
                                                 const char *rb, int64_t base, int64_t hi, int lane) {
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t i = base + lane_offset<MAPB>(lane, j);
    if (i < hi) {
      ua[j] = load_pattern<TA>(ra, i);
      ub[j] = load_pattern<TB>(rb, i);
      valid |= 1u << j;
    } else {
      ua[j] = 0xff800000u;
      ub[j] = 0xff800000u;
    }
  }
  return valid;
}

// ---------------------------------------------------------------- one wave step

template <bool CMP, bool BITS, bool W16, bool MAPB>
__device__ __forceinline__ void process_step(const uint32_t (&ua)[8], const uint32_t (&ub)[8],
                                             uint32_t valid, bool force_slow, int64_t base,
                                             int lane, int kint, WaveState &st, float *ba,
                                             float *bb, int *bi) {
  float xa[8], xb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    xa[j] = __uint_as_float(ua[j]);
    xb[j] = __uint_as_float(ub[j]);
  }
  const float ga = fmaxf(fmaxf(fmaxf(xa[0], xa[1]), fmaxf(xa[2], xa[3])),
                         fmaxf(fmaxf(xa[4], xa[5]), fmaxf(xa[6], xa[7])));
  const float gb = fmaxf(fmaxf(fmaxf(xb[0], xb[1]), fmaxf(xb[2], xb[3])),
                         fmaxf(fmaxf(xb[4], xb[5]), fmaxf(xb[6], xb[7])));

  if (CMP) {
    // move the exp2 reference when a logit outgrows it (rare after the first step)
    const float gm = fmaxf(ga, gb);
    if (ballot(gm > st.gate)) {
      const float wm = uniform(wave_max(gm));
      const float nh = wm * kL2E;
      const bool huge = fabsf(nh) >= 268435456.0f && isfinite(nh);
      const float nl = huge ? fmaf(wm, kL2E, -nh) : 0.0f;
      if (st.r2h > -INFINITY) {
        const double sc = exp2(((double)st.r2h + (double)st.r2l) - ((double)nh + (double)nl));
        st.s *= sc;
        st.d *= sc;
        st.f *= sc;
      }
      st.r2h = nh;
      st.r2l = nl;
      st.huge = st.huge || huge;
      st.gate = (nh + kRescaleLog2) * (1.0f / kL2E);
    }
  }

  // fast path: every element finite, |delta| <= 1/8
  float d[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) d[j] = xa[j] - xb[j];
  float sg = 0.0f, dg = 0.0f, fg = 0.0f;
  float sab = 0.0f, ssd = 0.0f, ssb = 0.0f, dmax = 0.0f;
  if (CMP) {
    float e[8], ed[8], ef[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      e[j] = __builtin_amdgcn_exp2f(fmaf(xa[j], kL2E, -st.r2h));
      ed[j] = e[j] * d[j];
      ef[j] = (ed[j] * d[j]) * phi_over_d2(d[j]);
    }
    sg = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
    dg = ((ed[0] + ed[1]) + (ed[2] + ed[3])) + ((ed[4] + ed[5]) + (ed[6] + ed[7]));
    fg = ((ef[0] + ef[1]) + (ef[2] + ef[3])) + ((ef[4] + ef[5]) + (ef[6] + ef[7]));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) dmax = fmaxf(dmax, fabsf(d[j]));
  if (BITS) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sab += fabsf(d[j]);
      ssd = fmaf(d[j], d[j], ssd);
      ssb = fmaf(xa[j], xa[j], ssb);
    }
  }
  bool ok = !force_slow;
  if (CMP) ok = ok && !st.huge && (dmax <= kPolyMax) && (dg == dg);
  if (BITS) ok = ok && isfinite(sab) && isfinite(ssd) && isfinite(ssb);

  if (ok) {
    if (CMP) {
      st.s += (double)sg;
      st.d += (double)dg;
      st.f += (double)fg;
    }
    if (BITS) {
      st.sab += (double)sab;
      st.ssd += (double)ssd;
      st.ssb += (double)ssb;
      st.max_abs = fmaxf(st.max_abs, dmax);
    }
  } else {
    // exact element-by-element path: special values and large differences
    float s2 = 0.0f, d2 = 0.0f, f2 = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!((valid >> j) & 1u)) continue;
      const float a = xa[j], b = xb[j];
      const bool fa = isfinite(a), fb = isfinite(b);
      if (BITS) {
        st.nfa += fa ? 0 : 1;
        st.nfb += fb ? 0 : 1;
        if (fa && fb) {
          const double dd = (double)a - (double)b;
          st.sab += fabs(dd);
          st.ssd += dd * dd;
          st.ssb += (double)a * (double)a;
          st.max_abs_d = fmax(st.max_abs_d, fabs(dd));
        }
      }
      if (CMP) {
        if (isnan(a) || isnan(b) || a == INFINITY || b == INFINITY) {
          st.n_bad++;
          continue;
        }
        if (a == -INFINITY) {
          st.n_ainf++;
          if (b == -INFINITY)
            st.n_binf++;
          else
            f2 += __builtin_amdgcn_exp2f(fmaf(b, kL2E, -st.r2h) - st.r2l);  // q mass where p = 0
          continue;
        }
        const float e = __builtin_amdgcn_exp2f(fmaf(a, kL2E, -st.r2h) - st.r2l);
        s2 += e;
        if (b == -INFINITY) {  // p > 0, q = 0: the full KL is infinite
          st.n_binf++;
          st.n_qzero++;
          f2 -= e;
          continue;
        }
        const float dj = a - b;
        const float ed = e * dj;
        d2 += ed;
        if (fabsf(dj) <= kPolyMax)
          f2 = fmaf(ed * dj, phi_over_d2(dj), f2);
        else  // e*phi = e*(delta - 1) + 2^(b*log2e - r2)
          f2 += fmaf(e, dj - 1.0f, __builtin_amdgcn_exp2f(fmaf(b, kL2E, -st.r2h) - st.r2l));
      }
    }
    if (CMP) {
      st.s += (double)s2;
      st.d += (double)d2;
      st.f += (double)f2;
    }
  }

  int idx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) idx[j] = (int)(base + lane_offset<MAPB>(lane, j));

  if (CMP) {
    // threshold from the first full step: the kint-th largest of the 64 lane maxima
    // (a full step has all 8 elements of every lane valid; the test is wave-uniform)
    if (!st.tau_set && !force_slow) {
      const uint32_t kg = rank_key(ga);
      uint32_t T = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t c = T | (1u << bit);
        if (__popcll(ballot(kg >= c)) >= kint) T = c;
      }
      st.tau_a = rank_key_inv(T);
      st.tau_i = 0x7fffffff;
      st.tau_set = true;
    }
    // top-k candidates: keys above the threshold go to the LDS buffer
    if (ballot(ga >= st.tau_a)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bool pass = ((valid >> j) & 1u) &&
                    (xa[j] > st.tau_a || (xa[j] == st.tau_a && idx[j] < st.tau_i));
        uint64_t m = ballot(pass);
        if (!m) continue;
        if (st.cnt + __popcll(m) > kCap) {
          flush_candidates(ba, bb, bi, st, kint);
          pass = ((valid >> j) & 1u) &&
                 (xa[j] > st.tau_a || (xa[j] == st.tau_a && idx[j] < st.tau_i));
          m = ballot(pass);
          if (!m) continue;
        }
        const int pos = st.cnt + prefix_count(m);
        if (pass) {
          ba[pos] = xa[j];
          bb[pos] = xb[j];
          bi[pos] = idx[j];
        }
        st.cnt += __popcll(m);
      }
      if (st.cnt >= kFlushAt) flush_candidates(ba, bb, bi, st, kint);
    }
    // candidate argmax, lowest index on ties (steps of a wave ascend in index)
    if (ballot(gb > st.bmax)) {
      const float wm = uniform(wave_max(gb));
      int li = 0x7fffffff;
#pragma unroll
      for (int j = 7; j >= 0; --j)
        if (((valid >> j) & 1u) && xb[j] == wm) li = idx[j];
      st.bmax = wm;
      st.bidx = uniform(wave_min(li));
    }
  }

  if (BITS) {
    uint64_t any = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t m = ballot(ua[j] != ub[j]);
      st.ndiff += __popcll(m);
      any |= m;
      uint32_t oa, ob;
      if (W16) {
        oa = ulp_order16(ua[j] >> 16);
        ob = ulp_order16(ub[j] >> 16);
      } else {
        oa = ulp_order32(ua[j]);
        ob = ulp_order32(ub[j]);
      }
      st.max_ulp = max(st.max_ulp, max(oa, ob) - min(oa, ob));
    }
    if (st.first < 0 && any) {
      int li = 0x7fffffff;
#pragma unroll
      for (int j = 7; j >= 0; --j)
        if (ua[j] != ub[j]) li = idx[j];
      st.first = uniform(wave_min(li));
    }
  }
}

// ---------------------------------------------------------------- kernel

template <int TA, int TB, bool CMP, bool BITS, bool VEC>
__global__ __launch_bounds__(kBlock) void k_row_stats(StreamArgs args) {
  constexpr bool MAPB = (TA == 1 && TB == 1);
  constexpr bool W16 = (TA == 1 && TB == 1);
  constexpr int SA = TA == 1 ? 2 : 4, SB = TB == 1 ? 2 : 4;
  __shared__ float s_ba[kWavesPerBlock][CMP ? kCap : 1];
  __shared__ float s_bb[kWavesPerBlock][CMP ? kCap : 1];
  __shared__ int s_bi[kWavesPerBlock][CMP ? kCap : 1];

  const int wid = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wid;
  const int64_t items = args.n * args.nchunks;
  if (item >= items) return;
  const int64_t row = item / args.nchunks;
  const int chunk = (int)(item - row * args.nchunks);
  const int64_t lo = (int64_t)chunk * args.chunk;
  const int64_t hi = min(args.v, lo + args.chunk);
  const char *ra = (const char *)args.a + row * args.lda * SA;
  const char *rb = (const char *)args.b + row * args.ldb * SB;
  float *ba = s_ba[wid];
  float *bb = s_bb[wid];
  int *bi = s_bi[wid];
  const int kint = args.kint;

  WaveState st;
  st.s = st.d = st.f = 0.0;
  st.r2h = -INFINITY;
  st.r2l = 0.0f;
  st.huge = false;
  st.gate = -INFINITY;
  st.bmax = -INFINITY;
  st.bidx = -1;
  st.tau_a = -INFINITY;
  st.tau_i = 0x7fffffff;
  st.cnt = 0;
  st.tau_set = false;
  st.n_bad = st.n_ainf = st.n_binf = st.n_qzero = 0;
  st.ndiff = 0;
  st.first = -1;
  st.max_ulp = 0;
  st.max_abs = 0.0f;
  st.max_abs_d = 0.0;
  st.sab = st.ssd = st.ssb = 0.0;
  st.nfa = st.nfb = 0;

  const int64_t nfull = (hi - lo) / kSpan;
  if (VEC) {
    if (nfull > 0) {
      Raw<TA, TB> cur, nxt;
      load_vec<TA, TB>(cur, ra, rb, lo, lane);
      for (int64_t sp = 0; sp < nfull; ++sp) {
        const int64_t base = lo + sp * kSpan;
        if (sp + 1 < nfull) load_vec<TA, TB>(nxt, ra, rb, base + kSpan, lane);
        uint32_t ua[8], ub[8];
        decode<TA, MAPB>(cur.a0, cur.a1, ua);
        decode<TB, MAPB>(cur.b0, cur.b1, ub);
        process_step<CMP, BITS, W16, MAPB>(ua, ub, 0xffu, false, base, lane, kint, st, ba, bb, bi);
        cur = nxt;
      }
    }
  } else {
    for (int64_t sp = 0; sp < nfull; ++sp) {
      const int64_t base = lo + sp * kSpan;
      uint32_t ua[8], ub[8];
      const uint32_t valid = load_checked<TA, TB, MAPB>(ua, ub, ra, rb, base, hi, lane);
      process_step<CMP, BITS, W16, MAPB>(ua, ub, valid, false, base, lane, kint, st, ba, bb, bi);
    }
  }
  if (lo + nfull * kSpan < hi) {
    const int64_t base = lo + nfull * kSpan;
    uint32_t ua[8], ub[8];
    const uint32_t valid = load_checked<TA, TB, MAPB>(ua, ub, ra, rb, base, hi, lane);
    process_step<CMP, BITS, W16, MAPB>(ua, ub, valid, true, base, lane, kint, st, ba, bb, bi);
  }

  // ---- wave totals, fixed order
  if (CMP) {
    if (st.cnt > kint) flush_candidates(ba, bb, bi, st, kint);
    wave_fence();
    const int64_t tk = item * kint;
    if (lane < st.cnt) {
      args.ta[tk + lane] = ba[lane];
      args.tb[tk + lane] = bb[lane];
      args.ti[tk + lane] = bi[lane];
    }
    const double S = wave_sum(st.s), D = wave_sum(st.d), F = wave_sum(st.f);
    const int nb = wave_sum(st.n_bad), na = wave_sum(st.n_ainf), nbi = wave_sum(st.n_binf),
              nq = wave_sum(st.n_qzero);
    if (lane == 0) {
      ChunkStats cs;
      cs.s = S;
      cs.d = D;
      cs.f = F;
      cs.r2 = st.r2h > -INFINITY ? (double)st.r2h + (double)st.r2l : -INFINITY;
      cs.bmax = st.bmax;
      cs.bidx = st.bidx;
      cs.cnt = st.cnt;
      cs.n_bad = nb;
      cs.n_ainf = na;
      cs.n_binf = nbi;
      cs.n_qzero = nq;
      cs.pad_ = 0;
      args.stats[item] = cs;
    }
  }
  if (BITS) {
    const double sab = wave_sum(st.sab), ssd = wave_sum(st.ssd), ssb = wave_sum(st.ssb);
    const int nfa = wave_sum(st.nfa), nfb = wave_sum(st.nfb);
    const uint32_t mu = wave_max(st.max_ulp);
    const double ma = wave_max(fmax((double)st.max_abs, st.max_abs_d));
    if (lane == 0) {
      ChunkBits cb;
      cb.ndiff = st.ndiff;
      cb.first = st.first;
      cb.nfa = nfa;
      cb.nfb = nfb;
      cb.max_ulp = mu;
      cb.pad_ = 0;
      cb.max_abs = ma;
      cb.sum_abs = sab;
      cb.ssd = ssd;
      cb.ssb = ssb;
      args.bits[item] = cb;
    }
  }
}

// ---------------------------------------------------------------- launcher

template <int TA, int TB, bool CMP, bool BITS>
static hipError_t launch_typed(const StreamArgs &a, bool vec, hipStream_t stream) {
  const int64_t items = a.n * a.nchunks;
  const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock));
  if (vec)
    hipLaunchKernelGGL((k_row_stats<TA, TB, CMP, BITS, true>), grid, dim3(kBlock), 0, stream, a);
  else
    hipLaunchKernelGGL((k_row_stats<TA, TB, CMP, BITS, false>), grid, dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

template <bool CMP, bool BITS>
static hipError_t launch_mode(const StreamArgs &a, int ta, int tb, bool vec, hipStream_t s) {
  if (ta == 0 && tb == 0) return launch_typed<0, 0, CMP, BITS>(a, vec, s);
  if (ta == 0 && tb == 1) return launch_typed<0, 1, CMP, BITS>(a, vec, s);
  if (ta == 1 && tb == 0) return launch_typed<1, 0, CMP, BITS>(a, vec, s);
  return launch_typed<1, 1, CMP, BITS>(a, vec, s);
}

hipError_t launch_row_stats(const StreamArgs &a, int ta, int tb, bool cmp, bool bits, bool vec,
                            hipStream_t stream) {
  if (a.n * a.nchunks == 0) return hipSuccess;
  if (cmp && bits) return launch_mode<true, true>(a, ta, tb, vec, stream);
  if (cmp) return launch_mode<true, false>(a, ta, tb, vec, stream);
  return launch_mode<false, true>(a, ta, tb, vec, stream);
}

}  // namespace lcmp
