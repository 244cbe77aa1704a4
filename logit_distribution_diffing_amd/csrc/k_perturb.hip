// k_perturb.hip -- precision perturbations for precision-knee experiments
// (page "在 agent 时代如何快速验证 kernel 对精度的影响", section 实验: keep only m
// fraction bits of an fp32 value with the exponent range unchanged, or round
// attention-weight-like values to fp8 e4m3, directly or after scaling by 448).
//
// Elementwise and HBM-bound: one block of 256 threads covers 1024 elements of
// one row, four per thread, with 16-byte (fp32) or 8-byte (bf16) accesses when
// the row is aligned and the tile is full.  Rounding is round to nearest, ties
// to even, done on the bit pattern: add half the dropped quantum minus one plus
// the lowest kept bit, then clear the dropped bits (a carry moves into the
// exponent, and past the largest finite value into infinity).
#include "common.hpp"
#include "launch.hpp"

namespace lcmp {

namespace {

constexpr int kPerturbTile = 1024;

// keep m (0..23) fraction bits of an fp32 pattern; inf and NaN pass unchanged
__device__ __forceinline__ uint32_t keep_bits(uint32_t u, int drop) {
  if ((u & 0x7f800000u) == 0x7f800000u || drop == 0) return u;
  const uint32_t low = (1u << drop) - 1u;
  const uint32_t bias = (low >> 1) + ((u >> drop) & 1u);
  return (u + bias) & ~low;
}

// OCP e4m3 (fn): 3 fraction bits, smallest exponent -6 (subnormal quantum
// 2^-9), largest finite 448, saturating; NaN passes unchanged
__device__ __forceinline__ float e4m3(float x) {
  if (x != x) return x;
  float r;
  if (fabsf(x) < 0x1p-6f)
    r = __builtin_rintf(x * 512.0f) * 0x1p-9f;  // exact scalings by powers of two
  else
    r = __uint_as_float(keep_bits(__float_as_uint(x), 20));
  return fminf(fmaxf(r, -448.0f), 448.0f);
}

template <int MODE>
__device__ __forceinline__ uint32_t perturb(uint32_t u, int drop) {
  if (MODE == 0) return keep_bits(u, drop);
  const float x = __uint_as_float(u);
  if (MODE == 1) return __float_as_uint(e4m3(x));
  // scaled: fp32 product, e4m3, fp32 quotient (correctly rounded division)
  return __float_as_uint(e4m3(x * 448.0f) / 448.0f);
}

template <int TS>
__device__ __forceinline__ uint32_t load_elem(const char *row, int64_t c) {
  if (TS == 1) return (uint32_t)(*(const uint16_t *)(row + 2 * c)) << 16;
  return *(const uint32_t *)(row + 4 * c);
}

// upper half of a pattern with at most 7 fraction bits; a NaN whose payload
// sits in the lower half keeps a quiet bit so that it stays a NaN
__device__ __forceinline__ uint32_t bf16_half(uint32_t u) {
  const bool nan = (u & 0x7fffffffu) > 0x7f800000u;
  return (u >> 16) | (nan ? 0x0040u : 0u);
}

template <int TD>
__device__ __forceinline__ void store_elem(char *row, int64_t c, uint32_t u) {
  if (TD == 1)
    *(uint16_t *)(row + 2 * c) = (uint16_t)bf16_half(u);
  else
    *(uint32_t *)(row + 4 * c) = u;
}

template <int TS, int TD, int MODE>
__global__ __launch_bounds__(256) void k_perturb(PerturbArgs a) {
  constexpr int ES = TS == 1 ? 2 : 4, ED = TD == 1 ? 2 : 4;
  const int64_t tile = blockIdx.x;
  const int64_t row = tile / a.tiles;
  const int64_t c0 = (tile - row * a.tiles) * kPerturbTile + 4 * (int64_t)threadIdx.x;
  const char *sr = (const char *)a.src + row * a.ld_src * ES;
  char *dr = (char *)a.dst + row * a.ld_dst * ED;
  const int drop = 23 - a.param;
  if (a.vec && c0 + 4 <= a.cols) {
    uint32_t u[4];
    if (TS == 1) {
      const u32x2 p = __builtin_nontemporal_load((const u32x2 *)(sr + 2 * c0));
      u[0] = p.x << 16;
      u[1] = p.x & 0xffff0000u;
      u[2] = p.y << 16;
      u[3] = p.y & 0xffff0000u;
    } else {
      const u32x4 p = __builtin_nontemporal_load((const u32x4 *)(sr + 4 * c0));
      u[0] = p.x;
      u[1] = p.y;
      u[2] = p.z;
      u[3] = p.w;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = perturb<MODE>(u[j], drop);
    if (TD == 1) {
      u32x2 q;
      q.x = bf16_half(u[0]) | (bf16_half(u[1]) << 16);
      q.y = bf16_half(u[2]) | (bf16_half(u[3]) << 16);
      __builtin_nontemporal_store(q, (u32x2 *)(dr + 2 * c0));
    } else {
      u32x4 q;
      q.x = u[0];
      q.y = u[1];
      q.z = u[2];
      q.w = u[3];
      __builtin_nontemporal_store(q, (u32x4 *)(dr + 4 * c0));
    }
  } else {
    for (int64_t c = c0; c < c0 + 4 && c < a.cols; ++c)
      store_elem<TD>(dr, c, perturb<MODE>(load_elem<TS>(sr, c), drop));
  }
}

template <int TS, int TD>
hipError_t launch_mode(const PerturbArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)(a.rows * a.tiles));
  if (a.mode == 0)
    hipLaunchKernelGGL((k_perturb<TS, TD, 0>), grid, dim3(256), 0, s, a);
  else if (a.mode == 1)
    hipLaunchKernelGGL((k_perturb<TS, TD, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_perturb<TS, TD, 2>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int64_t perturb_tiles(int64_t cols) { return (cols + kPerturbTile - 1) / kPerturbTile; }

hipError_t launch_perturb(const PerturbArgs &a, hipStream_t stream) {
  if (a.rows == 0 || a.cols == 0) return hipSuccess;
  if (a.ts == 0 && a.td == 0) return launch_mode<0, 0>(a, stream);
  if (a.ts == 0 && a.td == 1) return launch_mode<0, 1>(a, stream);
  if (a.ts == 1 && a.td == 0) return launch_mode<1, 0>(a, stream);
  return launch_mode<1, 1>(a, stream);
}

}  // namespace lcmp
