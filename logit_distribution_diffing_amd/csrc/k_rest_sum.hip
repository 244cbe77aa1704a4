// k_rest_sum.hip -- one-side streaming pass of the compact-record comparison
// (gfx950).
//
// A stored baseline record holds each row's top-k logits and the log of the
// mass outside them, so comparing a candidate against it needs only the
// candidate row (page "在 agent 时代如何快速验证 kernel 对精度的影响", section
// 先要有一个 ground truth: record the ground truth once, then compare every
// change against the record).  Of the candidate row this pass computes, per
// (row, chunk):
//   s     sum over the columns outside the row's head set H (the record's top-k
//         indices) of 2^((y - r) * log2e), against a wave-uniform reference r
//         that is the largest logit outside H seen so far (so the sum of the
//         rest is never lost under the head's much larger terms)
//   bmax, bidx   the largest logit over ALL columns and its lowest column
// and it flags NaN (through the sum) and +inf (through the reference).  The
// same pass over the baseline, with H its own top-k, gives the record's
// rest mass.
//
// One wave64 owns one (row, chunk) item.  A wave step covers 1 KiB per load
// instruction, two loads per lane: 512 fp32 columns or 1024 bf16 columns.  Load
// q of lane l holds columns [q*64*P + l*P, +P), P = 4 (fp32) or 8 (bf16).
// Aligned rows stream through a per-wave LDS ring (global_load_lds with the
// non-temporal hint, no registers held by loads in flight): R - 1 steps are in
// flight while one is read back and processed.  Measured at 10240 x 151936,
// the hint takes the stream from 5.96 to 6.70 TB/s; depths 3 to 6 are equal.  A register prefetch would be rotated with copies
// at every step, and those copies wait for the newest load.
//
// H has at most 64 members, one per lane; a step overlaps H in a handful of
// steps per row, found with one ballot per step, and only those steps take the
// masked branch.
#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"

#include <float.h>

namespace lcmp {

namespace {

constexpr int kRestR = 4;  // LDS ring slots per wave: one processed, the rest in flight

constexpr int kRestStepBytes = 2048;  // one wave step: two 1 KiB loads
static_assert((kRestR - 1) * 2 <= 63, "vector-memory counter range");
constexpr float kRestGate = kRescaleLog2 / kL2E;  // rescale slack in logit units

template <int T>
struct RestShape {
  static constexpr int ES = T == 1 ? 2 : 4;    // bytes per element
  static constexpr int P = 16 / ES;            // elements per 16-byte load
  static constexpr int EL = 2 * P;             // elements per lane per step
  static constexpr int SPAN = kWave * EL;      // columns per wave step
  static constexpr int HALF = kWave * P;       // columns per load instruction
};

struct RestBuf {
  u32x4 p0, p1;
};

struct RestState {
  double s;      // per lane
  float r, gate; // uniform reference and rescale gate (logit units)
  float bmax;    // uniform maximum over all columns
  int bidx;      // uniform lowest column of bmax, -1 if none
};

template <int T>
__device__ __forceinline__ void decode(const RestBuf &b, float (&y)[RestShape<T>::EL]) {
  const uint32_t w[8] = {b.p0.x, b.p0.y, b.p0.z, b.p0.w, b.p1.x, b.p1.y, b.p1.z, b.p1.w};
  if constexpr (T == 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      y[2 * i] = bf16_lo(w[i]);
      y[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = __uint_as_float(w[i]);
  }
}

// column offset of element j of a lane inside its step
template <int T>
__device__ __forceinline__ int col_of(int lane, int j) {
  using S = RestShape<T>;
  return (j / S::P) * S::HALF + lane * S::P + (j % S::P);
}

// bounds-checked loads of one step (ragged tail, unaligned rows): columns at
// or past hi read as -inf, which adds nothing to any statistic
template <int T>
__device__ __forceinline__ void load_checked(float (&y)[RestShape<T>::EL], const char *row,
                                             int base, int hi, int lane) {
#pragma unroll
  for (int j = 0; j < RestShape<T>::EL; ++j) {
    const int c = base + col_of<T>(lane, j);
    if (c < hi) {
      y[j] = T == 1 ? __uint_as_float((uint32_t)(*(const uint16_t *)(row + 2 * (int64_t)c)) << 16)
                    : *(const float *)(row + 4 * (int64_t)c);
    } else {
      y[j] = -INFINITY;
    }
  }
}

// v_max3_f32 on values straight from memory, without the NaN canonicalisation
// the compiler puts around fmaxf (a NaN flags its row through the sum anyway)
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

template <int N>
__device__ __forceinline__ float maxn(const float (&y)[N]) {
  static_assert(N == 8 || N == 16, "step width");
  float m = vmax3(vmax3(vmax3(y[0], y[1], y[2]), y[3], y[4]), vmax3(y[5], y[6], y[7]), y[7]);
  if constexpr (N == 16)
    m = vmax3(vmax3(vmax3(m, y[8], y[9]), vmax3(y[10], y[11], y[12]), y[13]), y[14], y[15]);
  return m;
}

// 2^d for d <= 0 to float accuracy (the integer part exactly), 0 below 2^-1100;
// used only when the reference moves, so no double polynomial is kept live
__device__ __forceinline__ double exp2_down(double d) {
  if (!(d > -1100.0)) return 0.0;
  const double n = floor(d);
  return ldexp((double)__builtin_amdgcn_exp2f((float)(d - n)), (int)n);
}

// ---------------------------------------------------------------- rare work

// new overall maximum: take the wave's largest value and its lowest column
template <int T>
__device__ __forceinline__ void take_argmax(RestState &st, const float (&y)[RestShape<T>::EL],
                                         float gm, int base, int lane) {
  const float wm = uniform(wave_max(gm));
  int c = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < RestShape<T>::EL; ++j)
    if (y[j] == wm) c = min(c, base + col_of<T>(lane, j));
  st.bmax = wm;
  st.bidx = uniform(wave_min(c));
}

// move the reference up to the wave's largest value outside the head set
__device__ __forceinline__ void rest_rescale(RestState &st, float gm) {
  const float wm = uniform(wave_max(gm));
  st.s *= exp2_down(((double)st.r - (double)wm) * (double)kL2E);
  st.r = wm;
  st.gate = uniform(wm + kRestGate);
}

// drop the head members that fall in this step (their value becomes -inf)
template <int T>
__device__ __forceinline__ void mask_head(float (&y)[RestShape<T>::EL], uint64_t hm, int hidx,
                                       int base, int lane) {
  using S = RestShape<T>;
  uint32_t m = 0;
  while (hm) {
    const int b = __builtin_ctzll(hm);
    hm &= hm - 1;
    const int c = __builtin_amdgcn_readlane(hidx, b) - base;
    const int q = c / S::HALF, rem = c - q * S::HALF;
    const int owner = rem / S::P;
    if (lane == owner) m |= 1u << (q * S::P + rem - owner * S::P);
  }
#pragma unroll
  for (int j = 0; j < S::EL; ++j)
    if ((m >> j) & 1u) y[j] = -INFINITY;
}

// ---------------------------------------------------------------- one step

template <int T>
__device__ __forceinline__ void rest_step(float (&y)[RestShape<T>::EL], int lo, int soff, int lane,
                                          int hidx, uint32_t hoff, RestState &st) {
  const int base = lo + soff;
  using S = RestShape<T>;
  float gm = maxn(y);
  if (ballot(gm > st.bmax)) take_argmax<T>(st, y, gm, base, lane);
  const uint64_t hm = ballot(hoff - (uint32_t)soff < (uint32_t)S::SPAN);
  if (hm) {
    mask_head<T>(y, hm, hidx, base, lane);
    gm = maxn(y);
  }
  if (ballot(gm > st.gate)) rest_rescale(st, gm);
  float e[S::EL];
#pragma unroll
  for (int j = 0; j < S::EL; ++j) e[j] = __builtin_amdgcn_exp2f((y[j] - st.r) * kL2E);
  // fixed pairwise order
#pragma unroll
  for (int w = 1; w < S::EL; w *= 2)
#pragma unroll
    for (int j = 0; j + w < S::EL; j += 2 * w) e[j] += e[j + w];
  st.s += (double)e[0];
}

template <int T, bool VEC>
__global__ __launch_bounds__(kBlock) void k_rest_sum(RestArgs a) {
  using S = RestShape<T>;
  __shared__ __attribute__((aligned(16))) char s_ring[kWavesPerBlock][VEC ? kRestR * kRestStepBytes : 16];
  const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int lane = lane_id();
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wid;
  if (item >= a.n * a.nchunks) return;
  const int64_t row = item / a.nchunks;
  const int chunk = (int)(item - row * a.nchunks);
  const int lo = (int)((int64_t)chunk * a.chunk);
  const int hi = (int)min(a.v, (int64_t)lo + a.chunk);
  const char *rp = (const char *)a.x + row * a.ldx * S::ES;
  // lane j holds head member j (or -1)
  const int hidx = lane < a.kh ? a.head[row * a.ldh + lane] : -1;

  RestState st;
  st.s = 0.0;
  st.r = -FLT_MAX;
  st.gate = -FLT_MAX;
  st.bmax = -INFINITY;
  st.bidx = -1;

  const int nfull = (hi - lo) / S::SPAN;
  uint32_t hoff;  // head member's column relative to the chunk start
  if constexpr (VEC) {
    const char *p = rp + (int64_t)lo * S::ES;
    char *ring = s_ring[wid];
    const uint32_t ring_lds = (uint32_t)(uintptr_t)ring;
    const uint32_t voff = 16u * (uint32_t)lane;
    const int npre = nfull < kRestR - 1 ? nfull : kRestR - 1;
#pragma unroll 1
    for (int q = 0; q < npre; ++q) {
      const char *g = p + (int64_t)q * kRestStepBytes;
      const uint32_t l = ring_lds + (uint32_t)(q * kRestStepBytes);
      dma_1k(g, voff, l);
      dma_1k(g + 1024, voff, l + 1024u);
    }
    // first use of the head index: its load was issued before the ring's
    hoff = (uint32_t)(hidx - lo);
    int rd = 0, wr = kRestR - 1;
#pragma unroll 1
    for (int sp = 0; sp < nfull; ++sp) {
      const int q = sp + kRestR - 1;
      if (q < nfull) {
        // slot wr was read back in the previous step, whose values are used
        // (so those reads have completed) before this copy is issued
        const char *g = p + (int64_t)q * kRestStepBytes;
        const uint32_t l = ring_lds + (uint32_t)(wr * kRestStepBytes);
        dma_1k(g, voff, l);
        dma_1k(g + 1024, voff, l + 1024u);
      }
      const int ahead = nfull - 1 - sp < kRestR - 1 ? nfull - 1 - sp : kRestR - 1;
      wait_step<2, kRestR - 1>(ahead);
      RestBuf b;
      const char *slot = ring + rd * kRestStepBytes;
      b.p0 = *(const u32x4 *)(slot + 16u * lane);
      b.p1 = *(const u32x4 *)(slot + 1024u + 16u * lane);
      float y[S::EL];
      decode<T>(b, y);
      rest_step<T>(y, lo, sp * S::SPAN, lane, hidx, hoff, st);
      rd = rd + 1 == kRestR ? 0 : rd + 1;
      wr = wr + 1 == kRestR ? 0 : wr + 1;
    }
  } else {
    hoff = (uint32_t)(hidx - lo);
#pragma unroll 1
    for (int sp = 0; sp < nfull; ++sp) {
      float y[S::EL];
      load_checked<T>(y, rp, lo + sp * S::SPAN, hi, lane);
      rest_step<T>(y, lo, sp * S::SPAN, lane, hidx, hoff, st);
    }
  }
  if (lo + nfull * S::SPAN < hi) {
    float y[S::EL];
    load_checked<T>(y, rp, lo + nfull * S::SPAN, hi, lane);
    rest_step<T>(y, lo, nfull * S::SPAN, lane, hidx, hoff, st);
  }

  const double tot = wave_sum(st.s);
  if (lane == 0) {
    RestChunk rc;
    rc.s = tot;
    rc.r = st.r;
    rc.bmax = st.bmax;
    rc.bidx = st.bidx;
    rc.pad_ = 0;
    a.out[item] = rc;
  }
}

template <int T, bool VEC>
hipError_t launch_typed(const RestArgs &a, hipStream_t s, const Timing &t) {
  const int64_t items = a.n * a.nchunks;
  const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock));
  hipExtLaunchKernelGGL((k_rest_sum<T, VEC>), grid, dim3(kBlock), 0, s, t.before, t.after, 0, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rest_sum(const RestArgs &a, int tx, bool vec, hipStream_t stream,
                           const Timing &t) {
  if (a.n * a.nchunks == 0) return record_empty(t, stream);
  if (tx == 1)
    return vec ? launch_typed<1, true>(a, stream, t) : launch_typed<1, false>(a, stream, t);
  return vec ? launch_typed<0, true>(a, stream, t) : launch_typed<0, false>(a, stream, t);
}

}  // namespace lcmp
