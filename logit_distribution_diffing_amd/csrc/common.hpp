// common.hpp -- device-side helpers and workspace records of liblcmp (gfx950).
//
// Layout decisions for CDNA4: one wave64 owns one (row, chunk) work item and
// streams it with 16-byte non-temporal loads; a 256-thread block is only a
// container of four independent waves, so the streaming kernel needs no
// barrier.  Per-lane accumulators are float for runs of 8 elements and
// double across runs; every cross-lane and cross-chunk reduction has a fixed
// order, so results are bit-identical from run to run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcmp {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kMaxK = 64;
constexpr int kSpan = kWave * 8;       // elements one wave covers per step (8 per lane)
constexpr int kMaxChunks = 64;         // chunks per row (one lane of the merge each)

// exp(x) is evaluated as exp2(x * kL2E - r2) with a wave-uniform reference r2
// (log2 units).  The finalize uses the same float constant, so the reference
// of the streamed sums and of the top-k terms agree exactly.
constexpr float kL2E = 1.44269504088896340736f;
constexpr double kLn2 = 0.69314718055994530942;
// lazily move the reference when a logit exceeds it by 2^24 (in exp2 units)
constexpr float kRescaleLog2 = 24.0f;
// |delta| bound of the polynomial for phi(d) = d + expm1(-d)
constexpr float kPolyMax = 0.125f;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));  // two 16-bit lanes of one register
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// --------------------------------------------------------------------- records

// One per (row, chunk): streamed softmax sums and counters.  s, d, f are
// sum e_i, sum e_i*delta_i and sum e_i*phi(delta_i) with e_i = 2^(a_i*kL2E - r2);
// w is the candidate's mass sum 2^(b_i*kL2E - r2), formed without cancellation.
struct ChunkStats {
  double s, d, f, w;
  double r2;     // reference in log2 units; -inf when the chunk held no finite logit
  float bmax;    // candidate maximum (-inf if none)
  int32_t bidx;  // lowest index of bmax, -1 if none
  int32_t cnt;   // top-k entries stored for this chunk
  int32_t n_bad, n_ainf, n_binf, n_qzero;
  int32_t pad_;
};

// One per (row, chunk) when bitwise statistics are requested.
struct ChunkBits {
  int64_t ndiff, first;  // first differing column, -1 if none
  int64_t nfa, nfb;
  uint32_t max_ulp, pad_;
  double max_abs;
  double sum_abs, ssd, ssb;
};

// Public per-row record (mirrors lcmp_bitdiff_row).
struct BitdiffRow {
  int64_t ndiff, first_diff, nonfinite_a, nonfinite_b;
  uint32_t max_ulp, pad_;
  double max_abs, sum_abs, sum_sq_diff, sum_sq_base, mean_abs, rel_l2;
};

// --------------------------------------------------------------------- lanes

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// lanes below this one whose bit is set in m
__device__ __forceinline__ int prefix_count(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <typename T>
__device__ __forceinline__ T uniform(T x) {
  return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Wave reductions without LDS traffic.  Inside each 16-lane row, four DPP
// exchanges pair lane l with l^1, l^2, then the mirror lane in its 8-lane half
// and in its row; every lane of a row then holds the row's total (the combine
// is commutative, so partners compute the same bits).  The four row totals
// are read out of lanes 0, 16, 32, 48 and combined in one fixed order, the same
// on every lane.  All 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i in each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i in each row

template <typename T>
struct Bits32 {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  template <int CTRL>
  static __device__ __forceinline__ T dpp(T x) {
    if constexpr (sizeof(T) == 4) {
      return __builtin_bit_cast(T, dpp32<CTRL>(__builtin_bit_cast(uint32_t, x)));
    } else {
      const uint64_t u = __builtin_bit_cast(uint64_t, x);
      const uint64_t lo = dpp32<CTRL>((uint32_t)u), hi = dpp32<CTRL>((uint32_t)(u >> 32));
      return __builtin_bit_cast(T, lo | (hi << 32));
    }
  }
  static __device__ __forceinline__ T lane(T x, int l) {
    if constexpr (sizeof(T) == 4) {
      return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
    } else {
      const uint64_t u = __builtin_bit_cast(uint64_t, x);
      const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
      const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
      return __builtin_bit_cast(T, lo | (hi << 32));
    }
  }
};

template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T x, Op op) {
  using B = Bits32<T>;
  x = op(x, B::template dpp<kDppXor1>(x));
  x = op(x, B::template dpp<kDppXor2>(x));
  x = op(x, B::template dpp<kDppHalfMirror>(x));
  x = op(x, B::template dpp<kDppMirror>(x));
  return op(op(B::lane(x, 0), B::lane(x, 16)), op(B::lane(x, 32), B::lane(x, 48)));
}

// The same combine over lanes 0 .. n-1 only (n uniform, 1 <= n <= 64): with
// few lanes (the chunks of a row) a chain of lane reads in lane order is
// cheaper than the full exchange; either way the order is fixed.
template <typename T, typename Op>
__device__ __forceinline__ T lanes_reduce(T x, int n, Op op) {
  if (n > 8) return wave_reduce(x, op);
  using B = Bits32<T>;
  T r = B::lane(x, 0);
  for (int l = 1; l < n; ++l) r = op(r, B::lane(x, l));
  return r;
}
template <typename T>
__device__ __forceinline__ T lanes_sum(T x, int n) {
  return lanes_reduce(x, n, [](T a, T b) { return a + b; });
}
__device__ __forceinline__ double lanes_max(double x, int n) {
  return lanes_reduce(x, n, [](double a, double b) { return fmax(a, b); });
}
__device__ __forceinline__ float lanes_max(float x, int n) {
  return lanes_reduce(x, n, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ uint32_t lanes_max(uint32_t x, int n) {
  return lanes_reduce(x, n, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ int lanes_min(int x, int n) {
  return lanes_reduce(x, n, [](int a, int b) { return a < b ? a : b; });
}
__device__ __forceinline__ int64_t lanes_min(int64_t x, int n) {
  return lanes_reduce(x, n, [](int64_t a, int64_t b) { return a < b ? a : b; });
}

__device__ __forceinline__ double wave_sum(double x) {
  return wave_reduce(x, [](double a, double b) { return a + b; });
}
__device__ __forceinline__ int64_t wave_sum(int64_t x) {
  return wave_reduce(x, [](int64_t a, int64_t b) { return a + b; });
}
__device__ __forceinline__ int wave_sum(int x) {
  return wave_reduce(x, [](int a, int b) { return a + b; });
}
__device__ __forceinline__ double wave_max(double x) {
  return wave_reduce(x, [](double a, double b) { return fmax(a, b); });
}
__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  return wave_reduce(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ int wave_min(int x) {
  return wave_reduce(x, [](int a, int b) { return a < b ? a : b; });
}
__device__ __forceinline__ int64_t wave_min(int64_t x) {
  return wave_reduce(x, [](int64_t a, int64_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ int wave_max(int x) {
  return wave_reduce(x, [](int a, int b) { return a > b ? a : b; });
}

// --------------------------------------------------------------------- values

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Monotone unsigned image of a float for ranking: -0 is first folded onto +0
// (they compare equal), then positive patterns get the sign bit set and
// negative ones are inverted.
__device__ __forceinline__ uint32_t rank_key(float x) {
  uint32_t u = __float_as_uint(x + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float rank_key_inv(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Ordered image used for ULP distances (no folding of -0: +0 and -0 are one
// unit apart).  Width 32 on fp32 patterns.
__device__ __forceinline__ uint32_t ulp_order32(uint32_t u) {
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}
// Width 16 on a bf16 pattern held in the low half.
__device__ __forceinline__ uint32_t ulp_order16(uint32_t h) {
  return (h & 0x8000u) ? (~h & 0xffffu) : (h | 0x8000u);
}

// phi(d) / d^2 = 1/2 - d/6 + d^2/24 - d^3/120 + ..., truncated after d^3; the
// dropped terms are below 7e-7 relative for |d| <= 1/8.
__device__ __forceinline__ float phi_over_d2(float d) {
  float p = fmaf(d, -1.0f / 120.0f, 1.0f / 24.0f);
  p = fmaf(d, p, -1.0f / 6.0f);
  return fmaf(d, p, 0.5f);
}

// psi(x) = x - log1p(x), the second-order remainder of log1p (x >= -1).
__device__ __forceinline__ double psi(double x) { return x - log1p(x); }

}  // namespace lcmp
