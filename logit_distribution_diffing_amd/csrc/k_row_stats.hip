// k_row_stats.hip -- the streaming pass of the logit comparison (gfx950).
//
// One wave64 owns one (row, chunk) item and reads each element pair of its
// chunk exactly once from HBM.  Per element pair (a = baseline, b = candidate
// logit) it keeps, against a wave-uniform exp2 reference r2:
//   s = sum e,  d = sum e*delta,  f = sum e*phi(delta)
// with e = 2^(a*log2e - r2), delta = a - b and phi(delta) = delta + expm1(-delta),
// and the candidate's mass w = sum 2^(b*log2e - r2).  The finalize forms
// KL(P||Q) = f/s - psi(E/s), E = f - d, from these sums, or d/s + ln(w/s) when
// the two normalisers are far apart (teacher-forced full-vocabulary KL of the
// page "在 agent 时代如何快速验证 kernel 对精度的影响", section 怎么比两个分布).
// Along the way it tracks the candidate argmax and the baseline top-k
// candidates (threshold filter into an LDS buffer, radix-select flushes), and
// optionally the bitwise statistics of the pair (differing patterns, first
// differing column, ULP distance, error norms; page "Kestrel_VLLM - 18",
// section 二, and page "海光 DCU 实测", sections 1 and 7).
//
// Element mapping inside one wave step of 512 elements: when either side is
// fp32, lane l takes elements [4l, 4l+4) and [256+4l, 256+4l+4), so each load
// instruction of the wave covers one contiguous run; when both sides are bf16,
// lane l takes [8l, 8l+8) with one 16-byte load per side.
//
// Code shape: the per-step work is inlined into the streaming loop (twice when
// it alternates two register sets), its remainder and the ragged last step.
// Rare work (moving the exp2 reference, the exact fp64 path for special values
// and large differences, top-k buffer flushes, argmax updates) sits behind
// wave-uniform branches so the common step is straight-line code.
#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

#include <float.h>
#include <math.h>

namespace lcmp {

// The candidate buffer holds kCapW entries (value, index).  Each half of a
// step appends at most 4 entries per lane whose group maximum passes the
// threshold; when that bound could overflow the buffer it is first reduced to
// kint <= 64 entries (64 + 256 <= kCapW), and after a step it is reduced
// whenever it holds more than kFlushAt.
constexpr int kCapW = 8 * kWave;  // 512
constexpr int kFlushAt = 128;
// Appends test the value alone: every element at or above the threshold
// value passes.

struct WaveState {
  // softmax sums of the fast path (per lane, double across 8-element runs)
  double s, d, f;
  // the same sums of the exact path, and there also the candidate's mass
  // wx = sum 2^(b*log2e - r2), each weight formed in double.  The candidate's
  // mass of the fast path is s - d + f (every term e * e^-delta with
  // |delta| <= 1/8, no cancellation), formed once per chunk.
  double sx, dx, fx, wx;
  // uniform exp2 reference r2h + r2l: r2l is 0 unless the logits are so large
  // (|r2h| >= 2^28) that one float cannot hold the reference within a unit;
  // such chunks take the exact path throughout
  float r2h, r2l, gate;
  float nr2h;  // -r2h, kept where the per-element multiply-add reads it
  int huge;    // r2l != 0 (uniform)
  int seen;    // a finite baseline logit was seen; until then the reference
               // follows the candidate (uniform)
  // candidate argmax (uniform)
  float bmax;
  int bidx;
  // top-k threshold key (uniform) and buffer fill
  float tau_a;
  // value an element must reach to be appended: tau_a itself in the step that
  // set it, the next float above it in later steps (later steps hold higher
  // columns only, so an element equal to tau_a ranks below the threshold
  // entry); tau_fresh marks a threshold set by a flush in the current step
  float tau_cmp;
  int tau_fresh;
  int tau_set, cnt;  // tau_set: the first full step has set a threshold
  int cbit;          // highest bit a column of the row can have
  // counters (uniform: ballot counts over the exact path)
  int n_bad, n_ainf, n_binf, n_qzero;
  // bitwise statistics
  int ndiff, first;  // uniform (a chunk holds fewer than 2^31 elements)
  uint32_t max_ulp;  // exact path (and, without the comparison, every pair)
  float max_abs;
  double max_abs_d, sab, ssd, ssb;
  int nfa, nfb;  // uniform, as the counters above
  // fast path with the comparison: signed differences of the ordered images,
  // their running maximum and minimum (|difference| < 2^31 there; bf16 pairs
  // keep one 16-bit lane per half of a word), and the per-lane count of
  // differing patterns (a count in a register: a ballot per element, whose
  // mask the scalar unit must wait for, measured slower)
  int omax, omin;
  s16x2 hmax, hmin;
  uint32_t ndl;
  // bf16 pairs: the differing counts of the low and high halves of the
  // words since the last fold, one 16-bit count per half
  uint32_t ndh;
  // Two constants the compiler must not see as constants, set once through
  // empty asm statements: 1 in each 16-bit half (a literal 1 turns the packed
  // minimum below into a compare and select per half), and log2(e) in a
  // vector register, so that the exponent's multiply-add reads the reference
  // from its scalar register directly (with the literal it copies the
  // reference into a vector register at every step).
  uint32_t one2;
  float l2e;
  // float partial sums of the fast path, added into the double sums every
  // kFold steps, before the reference moves and at the end of the chunk
  float ps, pd, pf, pab, psd, psb;
  int nstep;  // steps since the last fold (uniform)
  // one threshold below the reference gate, the top-k threshold and the
  // candidate maximum less a margin above kPolyMax: a step whose baseline
  // values all lie below it touches none of the three (uniform)
  float low;
};

constexpr int kFold = 4;

__device__ __forceinline__ void fold_partials(WaveState &st) {
  st.s += (double)st.ps;
  st.d += (double)st.pd;
  st.f += (double)st.pf;
  st.sab += (double)st.pab;
  st.ssd += (double)st.psd;
  st.ssb += (double)st.psb;
  st.ps = st.pd = st.pf = st.pab = st.psd = st.psb = 0.0f;
  st.ndl += (st.ndh & 0xffffu) + (st.ndh >> 16);
  st.ndh = 0u;
  st.nstep = 0;
}

__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// v_max3_f32 without the NaN canonicalisation the compiler adds around fmaxf
// on loaded values (a NaN in a row flags it through the sums anyway).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max3abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max8(const float (&x)[8]) {
  return max3f(max3f(max3f(x[0], x[1], x[2]), x[3], x[4]), max3f(x[5], x[6], x[7]), x[7]);
}
__device__ __forceinline__ float max8abs(const float (&x)[8]) {
  return max3abs(max3abs(max3abs(x[0], x[1], x[2]), x[3], x[4]), max3abs(x[5], x[6], x[7]), x[7]);
}
__device__ __forceinline__ uint32_t sad_u32(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_sad_u32 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// ---------------------------------------------------------------- top-k buffer

// The least float above x (x itself for NaN and +inf; above either zero, the
// least positive subnormal).
__device__ __forceinline__ float next_up(float x) {
  if (!(x < INFINITY)) return x;
  if (x == 0.0f) return __uint_as_float(1u);
  const uint32_t u = __float_as_uint(x);
  return __uint_as_float(x > 0.0f ? u + 1u : u - 1u);
}

// One candidate buffer entry; value and column side by side, so an append or
// a read is one 8-byte LDS access.
struct Cand {
  float v;
  int i;
};

// Reduce the wave's candidate buffer (cnt > kint (value, column) entries in
// LDS) to exactly the kint largest keys -- value descending, index ascending
// -- and raise the threshold to at most the kint-th key.  Whole wave, uniform
// control flow.  The entries are read into registers once (lane l holds
// entries l, l + 64, ...); the selection is a radix search from the top bit,
// two bits per round (three ballots per entry round, issued together, so
// their round trips to the scalar unit overlap: half the rounds of a one-bit
// search), which stops as soon as exactly kint keys lie at or above its
// prefix: those are the kint largest, and the prefix serves as the threshold
// (later elements have higher columns than every entry, so any value with
// kint entries at or above it will do).
// A16: the values are bf16, so every key ends in 16 zero bits (positive) or
// 16 one bits (negative) and the search stops at bit 16.
constexpr uint32_t kKeyFinite = 0x00800000u;  // rank_key(-FLT_MAX): the lowest finite value
template <bool A16>
__device__ __forceinline__ void flush_candidates(Cand *cb, WaveState &st, int kint) {
  constexpr int kRounds = kCapW / kWave;
  wave_fence();
  const int lane = lane_id();
  const int cnt = st.cnt;
  const int per = (cnt + kWave - 1) / kWave;
  uint32_t key[kRounds];
  int idx[kRounds];
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    const int e = lane + kWave * q;
    key[q] = 0u;  // below every stored key (the smallest, -inf, maps to 0x007fffff)
    idx[q] = 0x7fffffff;
    if (q < per && e < cnt) {
      const Cand c = cb[e];
      key[q] = rank_key(c.v);
      idx[q] = c.i;
    }
  }
  // kint-th largest value key, two bits at a time from the top: the largest
  // of the three extensions of T with at least kint keys at or above it;
  // early exit once the prefix T (a finite value, so that the threshold is
  // one) has exactly kint keys at or above it
  uint32_t T = 0;
  int nT = cnt;  // keys >= T: every stored key is above 0
  bool early = false;
#pragma unroll 1
  for (int bit = 30; bit >= (A16 ? 16 : 0); bit -= 2) {
    const uint32_t c1 = T | (1u << bit), c2 = T | (2u << bit), c3 = T | (3u << bit);
    int n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
      if (q < per) {
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
    if (nT == kint && T >= kKeyFinite) {
      early = true;
      break;
    }
  }
  if (A16 && !early && T < 0x80000000u) T |= 0xffffu;
  // After a full search T is the kint-th key; when more than kint entries lie
  // at or above it, the ties at T are cut by column.
  int isel = 0x7fffffff;  // ties at T are kept up to this column
  if (nT > kint) {
    int ngt = 0, neq = 0;
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
      if (q < per) {
        ngt += __popcll(ballot(key[q] > T));
        neq += __popcll(ballot(key[q] == T));
      }
    }
    const int need = kint - ngt;  // >= 1 entries taken among the ties at T
    if (neq > need) {
      // need-th smallest index among the ties
      uint32_t I = 0;
#pragma unroll 1
      for (int bit = st.cbit; bit >= 0; --bit) {
        const uint32_t c = I | (1u << bit);
        int n = 0;
#pragma unroll
        for (int q = 0; q < kRounds; ++q)
          if (q < per) n += __popcll(ballot(key[q] == T && (uint32_t)idx[q] < c));
        if (n < need) I = c;
      }
      isel = (int)I;
    }
  }
  // compaction in entry order; all entries are in registers, so the buffer
  // can be overwritten freely
  wave_fence();
  int fill = 0;
#pragma unroll
  for (int q = 0; q < kRounds; ++q) {
    if (q < per) {
      const bool kp = key[q] > T || (key[q] == T && idx[q] <= isel);
      const uint64_t m = ballot(kp);
      if (kp) {
        const int pos = fill + prefix_count(m);
        cb[pos] = Cand{rank_key_inv(key[q]), idx[q]};
      }
      fill += __popcll(m);
    }
  }
  wave_fence();
  st.cnt = fill;
  st.tau_a = rank_key_inv(T);
  st.tau_cmp = st.tau_a;
  st.tau_fresh = 1;
  st.tau_set = 1;
}

// ---------------------------------------------------------------- element mapping

template <bool MAPB>
__device__ __forceinline__ int lane_offset(int lane, int j) {
  if (MAPB) return 8 * lane + j;
  return (j < 4 ? 0 : 256) + 4 * lane + (j & 3);
}

template <int T>
__device__ __forceinline__ uint32_t load_pattern(const char *row, int i) {
  if (T == 1) return (uint32_t)(*(const uint16_t *)(row + 2 * i)) << 16;
  return *(const uint32_t *)(row + 4 * i);
}

// Raw registers of one wave step: one lane's 8 elements of each side, as
// 16-byte (fp32, or bf16 when both sides are bf16) or 8-byte (bf16) pieces.
// `p` is the wave's step pointer; each lane adds its own byte offset.
template <int T, bool MAPB>
struct Side;
template <bool MAPB>
struct Side<0, MAPB> {
  u32x4 p0, p1;
  __device__ __forceinline__ void load(const char *p, uint32_t lane) {
    p0 = __builtin_nontemporal_load((const u32x4 *)(p + 16u * lane));
    p1 = __builtin_nontemporal_load((const u32x4 *)(p + 1024u + 16u * lane));
  }
  __device__ __forceinline__ void load_lds(const char *p, uint32_t lane) {
    p0 = *(const u32x4 *)(p + 16u * lane);
    p1 = *(const u32x4 *)(p + 1024u + 16u * lane);
  }
  __device__ __forceinline__ void decode(uint32_t (&u)[8]) const {
    u[0] = p0.x; u[1] = p0.y; u[2] = p0.z; u[3] = p0.w;
    u[4] = p1.x; u[5] = p1.y; u[6] = p1.z; u[7] = p1.w;
  }
};
template <>
struct Side<1, false> {
  u32x2 p0, p1;
  __device__ __forceinline__ void load(const char *p, uint32_t lane) {
    p0 = __builtin_nontemporal_load((const u32x2 *)(p + 8u * lane));
    p1 = __builtin_nontemporal_load((const u32x2 *)(p + 512u + 8u * lane));
  }
  __device__ __forceinline__ void load_lds(const char *p, uint32_t lane) {
    p0 = *(const u32x2 *)(p + 8u * lane);
    p1 = *(const u32x2 *)(p + 512u + 8u * lane);
  }
  __device__ __forceinline__ void decode(uint32_t (&u)[8]) const {
    u[0] = p0.x << 16; u[1] = p0.x & 0xffff0000u;
    u[2] = p0.y << 16; u[3] = p0.y & 0xffff0000u;
    u[4] = p1.x << 16; u[5] = p1.x & 0xffff0000u;
    u[6] = p1.y << 16; u[7] = p1.y & 0xffff0000u;
  }
};
template <>
struct Side<1, true> {
  u32x4 p0;
  __device__ __forceinline__ void load(const char *p, uint32_t lane) {
    p0 = __builtin_nontemporal_load((const u32x4 *)(p + 16u * lane));
  }
  __device__ __forceinline__ void load_lds(const char *p, uint32_t lane) {
    p0 = *(const u32x4 *)(p + 16u * lane);
  }
  __device__ __forceinline__ void decode(uint32_t (&u)[8]) const {
    u[0] = p0.x << 16; u[1] = p0.x & 0xffff0000u;
    u[2] = p0.y << 16; u[3] = p0.y & 0xffff0000u;
    u[4] = p0.z << 16; u[5] = p0.z & 0xffff0000u;
    u[6] = p0.w << 16; u[7] = p0.w & 0xffff0000u;
  }
};

template <int TA, int TB>
struct Raw {
  static constexpr bool MAPB = (TA == 1 && TB == 1);
  Side<TA, MAPB> a;
  Side<TB, MAPB> b;
  __device__ __forceinline__ void load(const char *pa, const char *pb, uint32_t lane) {
    a.load(pa, lane);
    b.load(pb, lane);
  }
  __device__ __forceinline__ void load_lds(const char *pa, const char *pb, uint32_t lane) {
    a.load_lds(pa, lane);
    b.load_lds(pb, lane);
  }
};

// The four words of each side of a bf16 / bf16 step (element 2i in the low
// half of word i, element 2i + 1 in the high half); other pairs have none.
template <int TA, int TB>
__device__ __forceinline__ void raw_words(const Raw<TA, TB> &r, uint32_t (&wa)[4], uint32_t (&wb)[4]) {
  if constexpr (TA == 1 && TB == 1) {
    wa[0] = r.a.p0.x; wa[1] = r.a.p0.y; wa[2] = r.a.p0.z; wa[3] = r.a.p0.w;
    wb[0] = r.b.p0.x; wb[1] = r.b.p0.y; wb[2] = r.b.p0.z; wb[3] = r.b.p0.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) wa[i] = wb[i] = 0u;
  }
}
// The same words rebuilt from the element patterns of a checked load.
__device__ __forceinline__ void pack_words(const uint32_t (&u)[8], uint32_t (&w)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = (u[2 * i] >> 16) | (u[2 * i + 1] & 0xffff0000u);
}

// ---------------------------------------------------------------- LDS staging ring

// Launch shape of one instantiation.  With the LDS ring, the bytes a CU keeps
// in flight (waves x (ring depth - 1) x step bytes) bound the stream's rate:
// with a few microseconds of loaded HBM latency, 6 TB/s needs about 100 KB per
// CU in flight, so the ring is deep and the blocks are small enough that the
// 160 KB of LDS of a CU holds several of them.
// Ring depths (measured: three slots, two steps in flight, for every pair)
// and which pairs stage through LDS: on the corpus (fp32 / bf16) and stream
// (bf16 / bf16) shapes the register double buffer is faster when one side is
// fp32 (more waves fit), the ring when both sides are bf16.
constexpr int kRingFF = 3;     // fp32 / fp32: 4 KiB steps
constexpr int kRingFH = 3;     // one fp32 side: 3 KiB steps
constexpr int kRingHH = 3;     // bf16 / bf16: 2 KiB steps
constexpr int kRingWaves = 4;  // waves per block when staging through LDS
constexpr int kRingMask = 8;   // bit 2 * TA + TB set: that pair uses the ring (bf16 / bf16 only)
template <int TA, int TB, bool CMP, bool VEC>
struct Shape {
  static constexpr bool RING = VEC && CMP && ((kRingMask >> (2 * TA + TB)) & 1);
  static constexpr int SA = TA == 1 ? 2 : 4, SB = TB == 1 ? 2 : 4;
  static constexpr int kStepA = kSpan * SA, kStepB = kSpan * SB;
  static constexpr int kStep = kStepA + kStepB;
  // ring slots: one step processed, R - 1 in flight
  static constexpr int R = !RING                  ? 1
                           : (TA == 1 && TB == 1) ? kRingHH
                           : (TA == 0 && TB == 0) ? kRingFF
                                                  : kRingFH;
  static constexpr int W = RING ? kRingWaves : kWavesPerBlock;  // waves per block
  static_assert((R - 1) * (kStep / 1024) <= 63, "vector-memory counter range");
};


// Bounds-checked element loads (ragged tail, unaligned rows); positions past
// `hi` read as -inf on both sides and are masked out of every statistic.
template <int TA, int TB, bool MAPB>
__device__ __forceinline__ uint32_t load_checked(uint32_t (&ua)[8], uint32_t (&ub)[8], const char *ra,
                                                 const char *rb, int base, int hi, int lane) {
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int i = base + lane_offset<MAPB>(lane, j);
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

// ---------------------------------------------------------------- rare work

// 2^x in double for the exact path: x = k + f with k = rint(x), then
// e^(f ln 2) by its Taylor series to the 12th power (|f ln 2| <= 0.35, so the
// dropped terms are below 1e-14 relative).  0 below 2^-1075, +inf from 2^1024.
__device__ __forceinline__ double exp2_d(double x) {
  if (!(x > -1075.0)) return 0.0;
  if (x >= 1024.0) return INFINITY;
  const double k = rint(x);
  const double t = (x - k) * kLn2;
  double p = 1.0 / 479001600.0;  // 1/12!
  p = fma(p, t, 1.0 / 39916800.0);
  p = fma(p, t, 1.0 / 3628800.0);
  p = fma(p, t, 1.0 / 362880.0);
  p = fma(p, t, 1.0 / 40320.0);
  p = fma(p, t, 1.0 / 5040.0);
  p = fma(p, t, 1.0 / 720.0);
  p = fma(p, t, 1.0 / 120.0);
  p = fma(p, t, 1.0 / 24.0);
  p = fma(p, t, 1.0 / 6.0);
  p = fma(p, t, 0.5);
  p = fma(p, t, 1.0);
  p = fma(p, t, 1.0);
  return ldexp(p, (int)k);
}

// phi(d) = d + expm1(-d) = d^2 (1/2 - d/3! + d^2/4! - ...) in double for
// |d| <= 1/8, to the 10th power of d (dropped terms below 1e-15 relative).
__device__ __forceinline__ double phi_d(double d) {
  double p = 1.0 / 3628800.0;  // 1/10!
  p = fma(p, -d, 1.0 / 362880.0);
  p = fma(p, -d, 1.0 / 40320.0);
  p = fma(p, -d, 1.0 / 5040.0);
  p = fma(p, -d, 1.0 / 720.0);
  p = fma(p, -d, 1.0 / 120.0);
  p = fma(p, -d, 1.0 / 24.0);
  p = fma(p, -d, 1.0 / 6.0);
  p = fma(p, -d, 0.5);
  return d * d * p;
}

// Move the exp2 reference when a logit outgrows it (rare after the first step),
// or onto the chunk's first finite baseline logits.  The reference and the
// gate stay wave-uniform, in scalar registers.  Below 2^28 (log2 units) the
// reference is an integer, so moving it scales the sums by an exact power of
// two; above, it is the float product plus its rounding residual, and the
// fractional part of the shift goes through exp2 in float (relative error
// near 1e-7, common to all the sums).
__device__ __forceinline__ void rescale(WaveState &st, float gm) {
  fold_partials(st);
  const float wm = uniform(wave_max(gm));
  const float xh = wm * kL2E;
  const bool huge = fabsf(xh) >= 268435456.0f && isfinite(xh);
  const float nh = uniform(huge ? xh : ceilf(xh));
  const float nl = uniform(huge ? fmaf(wm, kL2E, -xh) : 0.0f);
  // before the first reference the sums are still 0; a shift below 2^-2048
  // (or undefined, with infinite references) clears them.  A move down only
  // happens before any fast-path sum was formed.
  double sc = 0.0;
  const double dd = ((double)st.r2h - (double)nh) + ((double)st.r2l - (double)nl);
  if (st.r2h > -INFINITY && dd > -2048.0) {
    const double k = floor(dd);
    const float fr = (float)(dd - k);
    // a move down (only onto the first baseline logits) is capped at 2^1000
    sc = ldexp(fr == 0.0f ? 1.0 : (double)__builtin_amdgcn_exp2f(fr), (int)fmin(k, 1000.0));
  }
  st.s *= sc;
  st.d *= sc;
  st.f *= sc;
  st.sx *= sc;
  st.dx *= sc;
  st.fx *= sc;
  st.wx *= sc;
  st.r2h = nh;
  st.nr2h = -nh;
  st.r2l = nl;
  st.huge = huge ? 1 : 0;
  st.gate = uniform((nh + kRescaleLog2) * (1.0f / kL2E));
}

// Column of element j of a lane inside its step (j may be any value in [0, 8)).
template <bool MAPB>
__device__ __forceinline__ int lane_offset_dyn(int lane, int j) {
  if (MAPB) return 8 * lane + j;
  return 4 * lane + j + (j >= 4 ? 252 : 0);
}

// ---------------------------------------------------------------- ULP distance

// Distance of two patterns in the ordered integer image: |ua - ub| when the
// signs agree, ma + mb + 1 (through zero) when they differ.  bf16 patterns sit
// in the upper half, so the same formula yields the bf16 distance << 16.
template <bool W16>
__device__ __forceinline__ uint32_t ulp_exact(uint32_t ua, uint32_t ub) {
  const uint32_t same = sad_u32(ua, ub);
  const uint32_t cross = ua + ub + (W16 ? 0x80010000u : 0x80000001u);
  return (int32_t)(ua ^ ub) < 0 ? cross : same;
}

// Signed ordered image of a pattern: magnitudes stay, negative patterns map
// to -(magnitude + one unit), so -0 sits one unit below +0 and the distance
// above is the absolute difference of two images.  For a pair with
// |a - b| <= 1/8 (both finite) a pair of opposite signs has both magnitudes
// at most 1/8, so the difference stays far inside 32 bits (and, for bf16,
// inside 16 bits).
__device__ __forceinline__ int32_t order32(uint32_t u) {
  return (int32_t)(u ^ ((uint32_t)((int32_t)u >> 31) & 0x7fffffffu));
}
// The same for the two bf16 patterns of one word, one 16-bit lane each.
__device__ __forceinline__ s16x2 order16x2(uint32_t w) {
  const s16x2 t = __builtin_bit_cast(s16x2, w) >> (s16x2)15;
  return __builtin_bit_cast(s16x2, w ^ (__builtin_bit_cast(uint32_t, t) & 0x7fff7fffu));
}

// ---------------------------------------------------------------- one wave step

template <bool CMP, bool BITS, bool W16, bool MAPB, bool A16>
__device__ __forceinline__ void process_step(const uint32_t (&ua)[8], const uint32_t (&ub)[8],
                                             const uint32_t (&wa)[4], const uint32_t (&wb)[4],
                                             uint32_t valid, bool tail, int base, int lane,
                                             int kint, WaveState &st, Cand *cb) {
  // bf16 pairs with the comparison: element 2i is the low half of word i of
  // wa / wb, element 2i + 1 the high half
  constexpr bool PACK = CMP && BITS && W16;
  constexpr bool ORD = CMP && BITS && !W16;
  float xa[8], xb[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    xa[j] = __uint_as_float(ua[j]);
    xb[j] = __uint_as_float(ub[j]);
  }
  float ga = 0.0f;
  bool hot = false;
  if (CMP) {
    ga = max8(xa);
    // The reference follows the baseline, so its weights e never underflow
    // because the candidate runs far above it; the candidate's weights, in
    // the exact path only, are formed in double.  Before the chunk's first
    // finite baseline logit the candidate sets the reference, which then
    // moves to the baseline, down if need be.  A step below st.low (always
    // passed before the first finite baseline logit) needs none of this.
    hot = ballot(ga >= st.low) != 0;
    if (hot) {
      const float gb = max8(xb);
      bool need;
      float gsel = ga;
      if (st.seen) {
        need = ballot(ga > st.gate) != 0;
      } else if (ballot(ga > -INFINITY)) {
        need = true;
        st.seen = 1;
      } else {
        need = ballot(gb > st.gate) != 0;
        gsel = gb;
      }
      if (need) rescale(st, gsel);
    }
  }

  // fast path: every element finite, |delta| <= 1/8.  In the ragged last
  // step the columns past the end enter it as a neutral pair: equal values
  // of zero weight (-FLT_MAX, whose exp2 is 0) and no square.
  float ya[8], yb[8], sq[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool vj = !tail || ((valid >> j) & 1u);
    ya[j] = vj ? xa[j] : -FLT_MAX;
    yb[j] = vj ? xb[j] : -FLT_MAX;
    sq[j] = vj ? xa[j] : 0.0f;
  }
  float d[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) d[j] = ya[j] - yb[j];
  const float dmax = max8abs(d);
  float sg = 0.0f, dg = 0.0f, fg = 0.0f;
  float sab = 0.0f, ssd = 0.0f, ssb = 0.0f;
  if (CMP) {
    // e*phi(delta) = (e*delta^2) * P(delta), P(d) = 1/2 - d/6 + d^2/24; the
    // dropped d^3/120 term is below 3.3e-5 of P for |d| <= 1/8.  One
    // accumulator per sum: four waves per SIMD hide the chain latency.
    float e = __builtin_amdgcn_exp2f(fmaf(ya[0], st.l2e, st.nr2h));
    sg = e;
    dg = e * d[0];
    fg = e * ((d[0] * d[0]) * fmaf(d[0], fmaf(d[0], 1.0f / 24.0f, -1.0f / 6.0f), 0.5f));
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      e = __builtin_amdgcn_exp2f(fmaf(ya[j], st.l2e, st.nr2h));
      const float q = (d[j] * d[j]) * fmaf(d[j], fmaf(d[j], 1.0f / 24.0f, -1.0f / 6.0f), 0.5f);
      sg += e;
      dg = fmaf(e, d[j], dg);
      fg = fmaf(e, q, fg);
    }
  }
  if (BITS) {
    sab = fabsf(d[0]);
    ssd = d[0] * d[0];
    ssb = sq[0] * sq[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) {
      sab += fabsf(d[j]);
      ssd += d[j] * d[j];
      ssb = fmaf(sq[j], sq[j], ssb);
    }
  }
  // Every special value reaches a NaN or an infinity in the checked sums:
  // with the comparison, a NaN or inf on either side makes delta NaN or
  // infinite (sab, or dg alone), a huge baseline makes sum a^2 infinite, and
  // |delta| <= 1/8 bounds sum delta^2.  With the bitwise statistics the one
  // test dmax * 2^127 + (sab + ssb) <= 2^124 holds only when |delta| <= 1/8
  // and sum a^2 <= 2^124, so kFold steps of float partials stay finite.
  // In the ragged last step a lane whose columns all lie past the end holds
  // only neutral pairs; before the chunk has a reference (every column so far
  // -inf on both sides) their weight 2^(-FLT_MAX*log2e + inf) would be +inf,
  // so such a step goes to the exact path, which skips masked columns.
  // (the wave-uniform part apart, so that the ballot is the compare's own mask)
  const bool uok = (!tail || st.r2h > -INFINITY || !CMP) && !(CMP && st.huge);
  bool okv = true;
  if (CMP && BITS)
    okv = fmaf(dmax, 0x1p127f, sab + ssb) <= 0x1p124f;
  else if (CMP)
    okv = (dmax <= kPolyMax) && (dg == dg);
  else if (BITS)
    okv = isfinite(sab + ssd + ssb);
  const bool ok = uok && okv;
  const uint64_t badm = ballot(!okv);
  const bool any_bad = !uok || badm != 0;

  // signed differences of the ordered images (bf16 pairs: two per word) and
  // their differing-pattern count, for every lane
  s16x2 od[4];
  if (PACK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) od[i] = order16x2(wa[i]) - order16x2(wb[i]);
    // min(difference, 1) in each unsigned 16-bit lane is one exactly when
    // the lane differs; four words add at most 4 to each half per step, and
    // the halves are folded into ndl every kFold steps, so the low half never
    // carries into the high one
    const uint32_t one2 = st.one2;
    uint32_t nz[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      nz[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, od[i]),
                                                                     __builtin_bit_cast(u16x2, one2)));
    st.ndh += nz[0] + nz[1] + nz[2] + nz[3];
  }

  if (ok) {
    if (CMP && BITS) {
      st.ps += sg;
      st.pd += dg;
      st.pf += fg;
      st.pab += sab;
      st.psd += ssd;
      st.psb += ssb;
    } else if (CMP) {
      st.s += (double)sg;
      st.d += (double)dg;
      st.f += (double)fg;
    } else if (BITS) {
      st.sab += (double)sab;
      st.ssd += (double)ssd;
      st.ssb += (double)ssb;
    }
    if (BITS) st.max_abs = max3f(st.max_abs, dmax, dmax);
    if (PACK) {
      const s16x2 m0 = __builtin_elementwise_max(od[0], od[1]);
      const s16x2 m1 = __builtin_elementwise_max(od[2], od[3]);
      const s16x2 n0 = __builtin_elementwise_min(od[0], od[1]);
      const s16x2 n1 = __builtin_elementwise_min(od[2], od[3]);
      st.hmax = __builtin_elementwise_max(st.hmax, __builtin_elementwise_max(m0, m1));
      st.hmin = __builtin_elementwise_min(st.hmin, __builtin_elementwise_min(n0, n1));
    }
    if (ORD) {
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const int32_t o0 = (int32_t)((uint32_t)order32(ua[j]) - (uint32_t)order32(ub[j]));
        const int32_t o1 = (int32_t)((uint32_t)order32(ua[j + 1]) - (uint32_t)order32(ub[j + 1]));
        st.omax = max(st.omax, max(o0, o1));
        st.omin = min(st.omin, min(o0, o1));
        // the ordered image is one-to-one: a difference is zero exactly when
        // the patterns agree
        st.ndl += min((uint32_t)o0, 1u) + min((uint32_t)o1, 1u);
      }
    }
  }
  if (CMP && BITS) {
    if (++st.nstep == kFold) fold_partials(st);
  }
  // exact element-by-element path for the lanes that are not ok: special
  // values, large differences, huge logits, ragged tails.  The branch is
  // taken by the whole wave (the lanes that are ok do nothing), so the
  // counters stay wave-uniform: ballots over the lanes at work.  The weights
  // are formed in double, where neither side under- or overflows.
  if (any_bad) {
    if (CMP && BITS && !ok) {
#pragma unroll
      for (int j = 0; j < 8; ++j) st.max_ulp = max(st.max_ulp, ulp_exact<W16>(ua[j], ub[j]));
    }
    const double r2d = (double)st.r2h + (double)st.r2l;
    // one element per trip (j is uniform): the double exponentials appear
    // once in the code rather than once per element
#pragma unroll 1
    for (int j = 0; j < 8; ++j) {
      float a = xa[0], b = xb[0];
#pragma unroll
      for (int t = 1; t < 8; ++t) {
        if (j == t) {
          a = xa[t];
          b = xb[t];
        }
      }
      const bool act = !ok && ((valid >> j) & 1u);
      if (ORD) {
        uint32_t pa = ua[0], pb = ub[0];
#pragma unroll
        for (int t = 1; t < 8; ++t) {
          if (j == t) {
            pa = ua[t];
            pb = ub[t];
          }
        }
        if (act && pa != pb) st.ndl += 1u;  // the lanes that are not ok
      }
      const bool fa = isfinite(a), fb = isfinite(b);
      if (BITS) {
        st.nfa += __popcll(ballot(act && !fa));
        st.nfb += __popcll(ballot(act && !fb));
        if (act && fa && fb) {
          const double dd = (double)a - (double)b;
          st.sab += fabs(dd);
          st.ssd += dd * dd;
          st.ssb += (double)a * (double)a;
          st.max_abs_d = fmax(st.max_abs_d, fabs(dd));
        }
      }
      if (CMP) {
        const bool bad = act && (isnan(a) || isnan(b) || a == INFINITY || b == INFINITY);
        const bool ainf = act && !bad && a == -INFINITY;
        const bool binf = act && !bad && b == -INFINITY;
        st.n_bad += __popcll(ballot(bad));
        st.n_ainf += __popcll(ballot(ainf));
        st.n_binf += __popcll(ballot(binf));
        st.n_qzero += __popcll(ballot(binf && !ainf));  // p > 0, q = 0: the full KL is infinite
        if (act && !bad) {
          if (ainf) {
            if (!binf) {  // q mass where p = 0
              const double eb = exp2_d((double)b * (double)kL2E - r2d);
              st.fx += eb;
              st.wx += eb;
            }
          } else {
            const double e = exp2_d((double)a * (double)kL2E - r2d);
            st.sx += e;
            if (binf) {
              st.fx -= e;
            } else {
              const double dj = (double)a - (double)b;  // exact
              const double eb = exp2_d((double)b * (double)kL2E - r2d);
              st.dx += e * dj;
              st.wx += eb;
              if (fabs(dj) <= (double)kPolyMax)
                st.fx += e * phi_d(dj);
              else  // e*phi = e*(delta - 1) + 2^(b*log2e - r2)
                st.fx += fma(e, dj - 1.0, eb);
            }
          }
        }
      }
    }
  }

  if (CMP && (hot || any_bad)) {
    const float gb = max8(xb);
    // top-k candidates: keys above the threshold go to the LDS buffer
    if (ballot(ga >= st.tau_a)) {
      // first full step: the kint-th largest of the 64 lane maxima bounds the
      // chunk's kint-th key from below
      if (!st.tau_set && !tail) {
        // (a prefix with exactly kint maxima at or above it bounds it too)
        const uint32_t kg = rank_key(ga);
        uint32_t T = 0;
        bool early = false;
#pragma unroll 1
        for (int bit = 30; bit >= (A16 ? 16 : 0); bit -= 2) {
          const uint32_t c1 = T | (1u << bit), c2 = T | (2u << bit), c3 = T | (3u << bit);
          const int n1 = __popcll(ballot(kg >= c1));
          const int n2 = __popcll(ballot(kg >= c2));
          const int n3 = __popcll(ballot(kg >= c3));
          int n = -1;
          if (n3 >= kint) {
            T = c3;
            n = n3;
          } else if (n2 >= kint) {
            T = c2;
            n = n2;
          } else if (n1 >= kint) {
            T = c1;
            n = n1;
          }
          if (n == kint && T >= kKeyFinite) {
            early = true;
            break;
          }
        }
        if (A16 && !early && T < 0x80000000u) T |= 0xffffu;
        st.tau_a = rank_key_inv(T);
        st.tau_cmp = st.tau_a;  // no column bound: equal values pass
        st.tau_set = 1;
      }
      if (st.tau_fresh) {
        st.tau_fresh = 0;
        st.tau_cmp = next_up(st.tau_a);
      }
      // at most 4 appends per passing lane and half step: make room first if
      // that could overflow
      const int npass = __popcll(ballot(ga >= st.tau_a));
      if (st.cnt + 4 * npass > kCapW) flush_candidates<A16>(cb, st, kint);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j == 4 && st.cnt + 4 * npass > kCapW) flush_candidates<A16>(cb, st, kint);
        // the value test alone: in the step of a flush an element equal to
        // the threshold value that ranks below the threshold entry (a higher
        // column) may ride along and lose in the next reduction
        const bool pass = ((valid >> j) & 1u) && xa[j] >= st.tau_cmp;
        const uint64_t m = ballot(pass);
        if (m) {
          if (pass) {
            const int pos = st.cnt + prefix_count(m);
            cb[pos] = Cand{xa[j], base + lane_offset<MAPB>(lane, j)};
          }
          st.cnt += __popcll(m);
        }
      }
      if (st.cnt > kFlushAt) flush_candidates<A16>(cb, st, kint);
    }
    // candidate argmax, lowest index on ties (steps of a wave ascend in index)
    if (ballot(gb > st.bmax)) {
      const float wm = uniform(wave_max(gb));
      int js = 8;  // first element of this lane equal to the maximum
#pragma unroll
      for (int j = 7; j >= 0; --j)
        if (((valid >> j) & 1u) && xb[j] == wm) js = j;
      const int li = js < 8 ? base + lane_offset_dyn<MAPB>(lane, js) : 0x7fffffff;
      st.bmax = wm;
      st.bidx = uniform(wave_min(li));
    }
    // A fast-path lane's candidate values stay within kPolyMax (plus the
    // rounding of delta) of its baseline values; a quarter covers both.
    st.low = st.seen ? fminf(fminf(st.gate, st.tau_a), st.bmax - 0.25f) : -INFINITY;
  }

  if (BITS) {
    if (PACK) {
      // first differing column, until one is found
      if (st.first < 0) {
        const uint32_t any = __builtin_bit_cast(uint32_t, od[0]) | __builtin_bit_cast(uint32_t, od[1]) |
                             __builtin_bit_cast(uint32_t, od[2]) | __builtin_bit_cast(uint32_t, od[3]);
        if (ballot(any != 0)) {
          int js = 8;  // first differing element of this lane
#pragma unroll
          for (int j = 7; j >= 0; --j)
            if (ua[j] != ub[j]) js = j;
          const int li = js < 8 ? base + lane_offset_dyn<MAPB>(lane, js) : 0x7fffffff;
          st.first = uniform(wave_min(li));
        }
      }
    } else if (ORD) {
      // first differing column, until one is found (the count is per lane)
      if (st.first < 0) {
        bool dj = false;
#pragma unroll
        for (int j = 0; j < 8; ++j) dj |= (ua[j] != ub[j]);
        if (ballot(dj)) {
          int js = 8;  // first differing element of this lane
#pragma unroll
          for (int j = 7; j >= 0; --j)
            if (ua[j] != ub[j]) js = j;
          const int li = js < 8 ? base + lane_offset_dyn<MAPB>(lane, js) : 0x7fffffff;
          st.first = uniform(wave_min(li));
        }
      }
    } else {
      // differing patterns (and, without the comparison, the ULP distance)
      uint64_t any = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint64_t m = ballot(ua[j] != ub[j]);
        st.ndiff += __popcll(m);
        any |= m;
        if (!CMP) st.max_ulp = max(st.max_ulp, ulp_exact<W16>(ua[j], ub[j]));
      }
      if (st.first < 0 && any) {
        int js = 8;  // first differing element of this lane
#pragma unroll
        for (int j = 7; j >= 0; --j)
          if (ua[j] != ub[j]) js = j;
        const int li = js < 8 ? base + lane_offset_dyn<MAPB>(lane, js) : 0x7fffffff;
        st.first = uniform(wave_min(li));
      }
    }
  }
}

// ---------------------------------------------------------------- kernel

template <int TA, int TB, bool CMP, bool BITS, bool VEC>
__global__ __launch_bounds__((Shape<TA, TB, CMP, VEC>::W * kWave))
__attribute__((amdgpu_waves_per_eu(4, 8))) void k_row_stats(StreamArgs args) {
  using SH = Shape<TA, TB, CMP, VEC>;
  constexpr bool MAPB = (TA == 1 && TB == 1);
  constexpr bool W16 = (TA == 1 && TB == 1);
  constexpr bool A16 = (TA == 1);  // baseline values (the top-k keys) are bf16
  constexpr int SA = SH::SA, SB = SH::SB;
  constexpr int kStepA = SH::kStepA, kStepB = SH::kStepB;
  constexpr bool RING = SH::RING;
  constexpr int R = SH::R, W = SH::W;
  constexpr int kRingBytes = RING ? R * SH::kStep : 16;
  __shared__ Cand s_cand[W][CMP ? kCapW : 1];
  __shared__ __attribute__((aligned(16))) char s_ring[W][kRingBytes];

  // every quantity derived from the wave id is uniform: keep it scalar
  const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int lane = lane_id();
  const int64_t item = (int64_t)blockIdx.x * W + wid;
  if (item >= args.n * args.nchunks) return;
  const int64_t row = item / args.nchunks;
  const int chunk = (int)(item - row * args.nchunks);
  // column indices fit in 32 bits (the vocabulary is below 2^31)
  const int lo = (int)((int64_t)chunk * args.chunk);
  const int hi = (int)min(args.v, (int64_t)lo + args.chunk);
  const char *ra = (const char *)args.a + row * args.lda * SA;
  const char *rb = (const char *)args.b + row * args.ldb * SB;
  Cand *cb = s_cand[wid];
  const int kint = args.kint;

  WaveState st;
  st.s = st.d = st.f = 0.0;
  st.sx = st.dx = st.fx = st.wx = 0.0;
  st.r2h = -INFINITY;
  st.nr2h = INFINITY;
  st.r2l = 0.0f;
  st.huge = 0;
  st.seen = 0;
  st.gate = -INFINITY;
  st.bmax = -INFINITY;
  st.bidx = -1;
  st.tau_a = -INFINITY;
  st.tau_cmp = -INFINITY;
  st.tau_fresh = 0;
  st.tau_set = 0;
  st.cnt = 0;
  st.cbit = args.v > 1 ? 63 - __builtin_clzll((unsigned long long)(args.v - 1)) : 0;
  st.n_bad = st.n_ainf = st.n_binf = st.n_qzero = 0;
  st.ndiff = 0;
  st.first = -1;
  st.max_ulp = 0;
  st.max_abs = 0.0f;
  st.max_abs_d = 0.0;
  st.sab = st.ssd = st.ssb = 0.0;
  st.nfa = st.nfb = 0;
  st.omax = st.omin = 0;
  st.hmax = st.hmin = (s16x2)0;
  st.ndl = 0u;
  st.ndh = 0u;
  asm volatile("" : "=v"(st.one2) : "0"(0x00010001u));
  asm volatile("" : "=v"(st.l2e) : "0"(kL2E));
  st.ps = st.pd = st.pf = st.pab = st.psd = st.psb = 0.0f;
  st.nstep = 0;
  st.low = -INFINITY;

  const int nfull = (hi - lo) / kSpan;
  if constexpr (RING) {
    // Full steps stream through a per-wave LDS ring: R - 1 steps are in
    // flight (global -> LDS, no registers held) while one is processed.  A
    // register-staged prefetch would have to be copied between register sets
    // at every step, and that copy waits for the newest load.
    constexpr int kStep = SH::kStep;
    constexpr int D = kStep / 1024;  // DMA operations per step
    char *ring = s_ring[wid];
    const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
    const char *pa = ra + (int64_t)lo * SA, *pb = rb + (int64_t)lo * SB;
    const uint32_t voff = 16u * (uint32_t)lane;
    const int npre = nfull < R - 1 ? nfull : R - 1;
#pragma unroll 1
    for (int q = 0; q < npre; ++q) {
      const uint32_t l = ring_lds + (uint32_t)(q * kStep);
      const char *ga = pa + (int64_t)q * kStepA, *gb = pb + (int64_t)q * kStepB;
#pragma unroll
      for (int c = 0; c < kStepA / 1024; ++c) dma_1k(ga + 1024 * c, voff, l + 1024u * c);
#pragma unroll
      for (int c = 0; c < kStepB / 1024; ++c) dma_1k(gb + 1024 * c, voff, l + kStepA + 1024u * c);
    }
    int rd = 0;      // slot of step sp
    int wr = R - 1;  // slot of step sp + R - 1
#pragma unroll 1
    for (int sp = 0; sp < nfull; ++sp) {
      const int q = sp + R - 1;
      if (q < nfull) {
        const uint32_t l = ring_lds + (uint32_t)(wr * kStep);
        const char *ga = pa + (int64_t)q * kStepA, *gb = pb + (int64_t)q * kStepB;
#pragma unroll
        for (int c = 0; c < kStepA / 1024; ++c) dma_1k(ga + 1024 * c, voff, l + 1024u * c);
#pragma unroll
        for (int c = 0; c < kStepB / 1024; ++c) dma_1k(gb + 1024 * c, voff, l + kStepA + 1024u * c);
      }
      // steps issued after this one
      const int ahead = nfull - 1 - sp < R - 1 ? nfull - 1 - sp : R - 1;
      wait_step<D, R - 1>(ahead);
      Raw<TA, TB> cur;
      const char *slot = ring + rd * kStep;
      cur.load_lds(slot, slot + kStepA, (uint32_t)lane);
      uint32_t ua[8], ub[8], wa[4], wb[4];
      cur.a.decode(ua);
      cur.b.decode(ub);
      raw_words(cur, wa, wb);
      process_step<CMP, BITS, W16, MAPB, A16>(ua, ub, wa, wb, 0xffu, false, lo + sp * kSpan, lane,
                                              kint, st, cb);
      rd = rd + 1 == R ? 0 : rd + 1;
      wr = wr + 1 == R ? 0 : wr + 1;
    }
  } else if constexpr (VEC) {
    // Two register sets used in turn: while one step is processed the other
    // set's loads are in flight, and nothing is copied between the sets.  The
    // prefetch is unconditional (past the end the last step is fetched again):
    // a load under a branch makes the wait before a use a full drain of the
    // memory counter.
    const char *pa = ra + (int64_t)lo * SA, *pb = rb + (int64_t)lo * SB;
    Raw<TA, TB> r0, r1;
    auto fetch = [&](Raw<TA, TB> &r, int s) {
      r.load(pa + (int64_t)s * kStepA, pb + (int64_t)s * kStepB, (uint32_t)lane);
    };
    auto step = [&](const Raw<TA, TB> &r, int s) {
      uint32_t ua[8], ub[8], wa[4], wb[4];
      r.a.decode(ua);
      r.b.decode(ub);
      raw_words(r, wa, wb);
      process_step<CMP, BITS, W16, MAPB, A16>(ua, ub, wa, wb, 0xffu, false, lo + s * kSpan, lane,
                                              kint, st, cb);
    };
    if (nfull > 0) fetch(r0, 0);
    int sp = 0;
#pragma unroll 1
    for (; sp + 1 < nfull; sp += 2) {
      fetch(r1, sp + 1);
      step(r0, sp);
      fetch(r0, sp + 2 < nfull ? sp + 2 : sp + 1);
      step(r1, sp + 1);
    }
    if (sp < nfull) step(r0, sp);
  } else {
#pragma unroll 1
    for (int sp = 0; sp < nfull; ++sp) {
      const int base = lo + sp * kSpan;
      uint32_t ua[8], ub[8], wa[4], wb[4];
      const uint32_t valid = load_checked<TA, TB, MAPB>(ua, ub, ra, rb, base, hi, lane);
      pack_words(ua, wa);
      pack_words(ub, wb);
      process_step<CMP, BITS, W16, MAPB, A16>(ua, ub, wa, wb, valid, false, base, lane, kint, st, cb);
    }
  }
  if (lo + nfull * kSpan < hi) {
    const int base = lo + nfull * kSpan;
    uint32_t ua[8], ub[8], wa[4], wb[4];
    const uint32_t valid = load_checked<TA, TB, MAPB>(ua, ub, ra, rb, base, hi, lane);
    pack_words(ua, wa);
    pack_words(ub, wb);
    process_step<CMP, BITS, W16, MAPB, A16>(ua, ub, wa, wb, valid, true, base, lane, kint, st, cb);
  }
  if (CMP && BITS) fold_partials(st);

  // ---- wave totals, fixed order.  The output pointers are read from the
  // argument segment here rather than held in scalar registers through the loop.
  const StreamArgs &late = *(const StreamArgs *)__builtin_amdgcn_kernarg_segment_ptr();
  if (CMP) {
    if (st.cnt > kint) flush_candidates<A16>(cb, st, kint);
    wave_fence();
    const int64_t tk = item * kint;
    if (lane < st.cnt) {
      const Cand c = cb[lane];
      late.ta[tk + lane] = c.v;
      late.ti[tk + lane] = c.i;
    }
    const double S = wave_sum(st.s + st.sx), D = wave_sum(st.d + st.dx),
                 F = wave_sum(st.f + st.fx);
    const double Wc = wave_sum(((st.s - st.d) + st.f) + st.wx);
    const int nb = st.n_bad, na = st.n_ainf, nbi = st.n_binf, nq = st.n_qzero;
    if (lane == 0) {
      ChunkStats cs;
      cs.s = S;
      cs.d = D;
      cs.f = F;
      cs.w = Wc;
      cs.r2 = st.r2h > -INFINITY ? (double)st.r2h + (double)st.r2l : -INFINITY;
      cs.bmax = st.bmax;
      cs.bidx = st.bidx;
      cs.cnt = st.cnt;
      cs.n_bad = nb;
      cs.n_ainf = na;
      cs.n_binf = nbi;
      cs.n_qzero = nq;
      cs.pad_ = 0;
      late.stats[item] = cs;
    }
  }
  if (BITS) {
    const double sab = wave_sum(st.sab), ssd = wave_sum(st.ssd), ssb = wave_sum(st.ssb);
    const int nfa = st.nfa, nfb = st.nfb;
    // fast-path ULP distances: the larger of the maximum and minus the minimum
    // of the image differences (0 without the comparison)
    uint32_t close;
    if (W16) {
      const int m = max(max((int)st.hmax.x, (int)st.hmax.y), -min((int)st.hmin.x, (int)st.hmin.y));
      close = (uint32_t)m;
    } else {
      close = (uint32_t)max(st.omax, -st.omin);
    }
    const uint32_t mu = max(wave_max(st.max_ulp) >> (W16 ? 16 : 0), wave_max(close));
    const int ndiff = st.ndiff + wave_sum((int)st.ndl);
    const double ma = wave_max(fmax((double)st.max_abs, st.max_abs_d));
    if (lane == 0) {
      ChunkBits cb;
      cb.ndiff = ndiff;
      cb.first = st.first;
      cb.nfa = nfa;
      cb.nfb = nfb;
      cb.max_ulp = mu;
      cb.pad_ = 0;
      cb.max_abs = ma;
      cb.sum_abs = sab;
      cb.ssd = ssd;
      cb.ssb = ssb;
      late.bits[item] = cb;
    }
  }
}

// ---------------------------------------------------------------- launcher

template <int TA, int TB, bool CMP, bool BITS, bool VEC>
static void launch_shape(const StreamArgs &a, hipStream_t stream, const Timing &t) {
  constexpr int W = Shape<TA, TB, CMP, VEC>::W;
  const int64_t items = a.n * a.nchunks;
  const dim3 grid((unsigned)((items + W - 1) / W));
  hipExtLaunchKernelGGL((k_row_stats<TA, TB, CMP, BITS, VEC>), grid, dim3(W * kWave), 0, stream,
                        t.before, t.after, 0, a);
}

template <int TA, int TB, bool CMP, bool BITS>
static hipError_t launch_typed(const StreamArgs &a, bool vec, hipStream_t stream, const Timing &t) {
  if (vec)
    launch_shape<TA, TB, CMP, BITS, true>(a, stream, t);
  else
    launch_shape<TA, TB, CMP, BITS, false>(a, stream, t);
  return hipGetLastError();
}

template <bool CMP, bool BITS>
static hipError_t launch_mode(const StreamArgs &a, int ta, int tb, bool vec, hipStream_t s,
                              const Timing &t) {
  if (ta == 0 && tb == 0) return launch_typed<0, 0, CMP, BITS>(a, vec, s, t);
  if (ta == 0 && tb == 1) return launch_typed<0, 1, CMP, BITS>(a, vec, s, t);
  if (ta == 1 && tb == 0) return launch_typed<1, 0, CMP, BITS>(a, vec, s, t);
  return launch_typed<1, 1, CMP, BITS>(a, vec, s, t);
}

hipError_t launch_row_stats(const StreamArgs &a, int ta, int tb, bool cmp, bool bits, bool vec,
                            hipStream_t stream, const Timing &t) {
  if (a.n * a.nchunks == 0) return record_empty(t, stream);
  if (cmp && bits) return launch_mode<true, true>(a, ta, tb, vec, stream, t);
  if (cmp) return launch_mode<true, false>(a, ta, tb, vec, stream, t);
  return launch_mode<false, true>(a, ta, tb, vec, stream, t);
}

}  // namespace lcmp
