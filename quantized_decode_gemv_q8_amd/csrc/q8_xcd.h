// XCD placement helpers shared by the split-K combines of the Q8_0 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// Id of the XCD this wave runs on (the XCC_ID hardware register; its low
// four bits).
__device__ __forceinline__ uint32_t xcd_id() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 15u;
}

// The split-K counter of a tile whose contributors are placed on one XCD is
// 64 bits: the number of contributors in bits 0-14, a count of contributors
// that report an XCD numbered 8 or above from bit 15, and a 6-bit count per
// XCD x at bit 16 + 6x.  A contributor on XCD x adds xcd_increment(x).
__device__ __forceinline__ uint64_t xcd_increment(uint32_t x) {
  return 1ull + (x < 8 ? 1ull << (16 + 6 * x) : 1ull << 15);
}

// Whether the contributor that brought the counter from `prev` to
// `prev + xcd_increment(x)` completed the tile's n contributions.
__device__ __forceinline__ bool xcd_count_done(uint64_t prev, uint64_t n) { return (prev & 0x7fffu) == n - 1; }

// For the contributor that completed the count: whether every one of the n
// contributors counted on its own XCD x.
__device__ __forceinline__ bool xcd_all_here(uint64_t prev, uint32_t x, uint64_t n) {
  return x < 8 && prev + xcd_increment(x) == n + (n << (16 + 6 * x));
}

}  // namespace q8
