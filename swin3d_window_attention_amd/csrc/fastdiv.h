// Division by a divisor fixed for a launch, as a multiply and a shift.
//
// floor(n / d) for 0 <= n < 2^31 as (n * mul) >> shr: with l = ceil(log2 d),
// shr = 31 + l and mul = ceil(2^shr / d), the product error stays below one
// step of n (Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, Theorem 4.2 with N = 31). The host computes
// (mul, shr) once per plan; the kernels divide with one 32 x 32 -> 64-bit
// multiply and a shift.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fastdiv {

struct FastDiv {
  uint32_t mul, shr;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint32_t shr = 31 + l;
  return FastDiv{(uint32_t)(((uint64_t(1) << shr) + d - 1) / d), shr};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)n * f.mul) >> f.shr);
}

}  // namespace fastdiv
