// k_read_probe.hip -- a read-only stream over the comparison's inputs, for
// measuring the read rate the hardware reaches on exactly the comparison's
// access pattern (gfx950).  Not part of the comparison: it computes nothing
// but an XOR of the words it reads, which it writes once per wave so the
// loads cannot be dropped.
//
// The decomposition is the streaming pass's: one wave64 per (row, chunk) with
// the same chunk length, steps of 512 elements of each side, lane l holding
// the same 8 elements of a step (one or two 16-byte non-temporal loads per
// side), the next step's loads issued before the current step is consumed
// (two register sets used in turn), and the ragged last step read with
// bounds-checked loads.
#include "common.hpp"
#include "launch.hpp"

namespace lcmp {

namespace {

// S = bytes per element; PAIR16: both sides bf16 (lane l holds elements
// [8l, 8l+8) of a step); otherwise lane l holds [4l, 4l+4) and [256+4l, +4).
template <int S, bool PAIR16>
struct ProbeSide;
template <bool PAIR16>
struct ProbeSide<4, PAIR16> {
  u32x4 p0, p1;
  __device__ __forceinline__ void load(const char *p, uint32_t lane) {
    p0 = __builtin_nontemporal_load((const u32x4 *)(p + 16u * lane));
    p1 = __builtin_nontemporal_load((const u32x4 *)(p + 1024u + 16u * lane));
  }
  __device__ __forceinline__ uint32_t fold() const {
    return p0.x ^ p0.y ^ p0.z ^ p0.w ^ p1.x ^ p1.y ^ p1.z ^ p1.w;
  }
};
template <>
struct ProbeSide<2, false> {
  u32x2 p0, p1;
  __device__ __forceinline__ void load(const char *p, uint32_t lane) {
    p0 = __builtin_nontemporal_load((const u32x2 *)(p + 8u * lane));
    p1 = __builtin_nontemporal_load((const u32x2 *)(p + 512u + 8u * lane));
  }
  __device__ __forceinline__ uint32_t fold() const { return p0.x ^ p0.y ^ p1.x ^ p1.y; }
};
template <>
struct ProbeSide<2, true> {
  u32x4 p0;
  __device__ __forceinline__ void load(const char *p, uint32_t lane) {
    p0 = __builtin_nontemporal_load((const u32x4 *)(p + 16u * lane));
  }
  __device__ __forceinline__ uint32_t fold() const { return p0.x ^ p0.y ^ p0.z ^ p0.w; }
};

template <int SA, int SB>
struct ProbeRaw {
  static constexpr bool PAIR16 = SA == 2 && SB == 2;
  ProbeSide<SA, PAIR16> a;
  ProbeSide<SB, PAIR16> b;
};

template <int SA, int SB>
__global__ __launch_bounds__(kBlock) void k_read_probe(StreamArgs args, uint32_t *sink) {
  constexpr int kStepA = kSpan * SA, kStepB = kSpan * SB;
  const int wid = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const uint32_t lane = (uint32_t)lane_id();
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + wid;
  if (item >= args.n * args.nchunks) return;
  const int64_t row = item / args.nchunks;
  const int chunk = (int)(item - row * args.nchunks);
  const int lo = (int)((int64_t)chunk * args.chunk);
  const int hi = (int)min(args.v, (int64_t)lo + args.chunk);
  const char *pa = (const char *)args.a + (row * args.lda + lo) * SA;
  const char *pb = (const char *)args.b + (row * args.ldb + lo) * SB;
  const int nfull = (hi - lo) / kSpan;
  uint32_t acc = 0;
  ProbeRaw<SA, SB> r0, r1;
  auto fetch = [&](ProbeRaw<SA, SB> &r, int s) {
    r.a.load(pa + (int64_t)s * kStepA, lane);
    r.b.load(pb + (int64_t)s * kStepB, lane);
  };
  if (nfull > 0) fetch(r0, 0);
  int sp = 0;
#pragma unroll 1
  for (; sp + 1 < nfull; sp += 2) {
    fetch(r1, sp + 1);
    acc ^= r0.a.fold() ^ r0.b.fold();
    fetch(r0, sp + 2 < nfull ? sp + 2 : sp + 1);
    acc ^= r1.a.fold() ^ r1.b.fold();
  }
  if (sp < nfull) acc ^= r0.a.fold() ^ r0.b.fold();
  // ragged last step: the same 8 elements per lane, bounds-checked
  const int base = nfull * kSpan;
  if (lo + base < hi) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = base + (SA == 2 && SB == 2 ? (int)(8 * lane) + j
                                               : (j < 4 ? 0 : 256) + (int)(4 * lane) + (j & 3));
      if (lo + i < hi) {
        acc ^= SA == 2 ? (uint32_t)((const uint16_t *)pa)[i] : ((const uint32_t *)pa)[i];
        acc ^= SB == 2 ? (uint32_t)((const uint16_t *)pb)[i] : ((const uint32_t *)pb)[i];
      }
    }
  }
  acc = wave_reduce(acc, [](uint32_t x, uint32_t y) { return x ^ y; });
  if (lane == 0) sink[item] = acc;
}

template <int SA, int SB>
hipError_t launch_probe_typed(const StreamArgs &a, uint32_t *sink, hipStream_t s, const Timing &t) {
  const int64_t items = a.n * a.nchunks;
  const dim3 grid((unsigned)((items + kWavesPerBlock - 1) / kWavesPerBlock));
  hipExtLaunchKernelGGL((k_read_probe<SA, SB>), grid, dim3(kBlock), 0, s, t.before, t.after, 0, a,
                        sink);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_read_probe(const StreamArgs &a, int ta, int tb, uint32_t *sink,
                             hipStream_t s, const Timing &t) {
  if (a.n * a.nchunks == 0) return record_empty(t, s);
  if (ta == 0 && tb == 0) return launch_probe_typed<4, 4>(a, sink, s, t);
  if (ta == 0 && tb == 1) return launch_probe_typed<4, 2>(a, sink, s, t);
  if (ta == 1 && tb == 0) return launch_probe_typed<2, 4>(a, sink, s, t);
  return launch_probe_typed<2, 2>(a, sink, s, t);
}

}  // namespace lcmp
