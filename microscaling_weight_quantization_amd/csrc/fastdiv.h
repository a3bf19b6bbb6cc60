// Unsigned 32-bit division by a divisor that is fixed for a whole launch.
//
// The kernels split a flat workgroup or step index into (row, segment) before
// their first load.  A plain `/` by a run-time value compiles to a float
// reciprocal plus correction steps on the vector unit, which sits in front of
// every wave's first load.  Instead the host computes, once per launch, the
// constants of the method of T. Granlund and P. L. Montgomery ("Division by
// invariant integers using multiplication", PLDI 1994, section 4):
//
//   l = ceil(log2 d),  m = floor(2^32 (2^l - d) / d) + 1   (m < 2^32 for d >= 1),
//   n / d = (mulhi(m, n) + n) >> l   for every 32-bit n,
//
// where the sum is formed in 64 bits, so the quotient costs one multiply-high,
// one add and one shift -- scalar instructions when n is uniform.
//
// Plain C++ (constexpr, no HIP types): the kernels use it, and so does a host
// test that checks the quotient against `/`.
#pragma once

#include <stdint.h>

struct MxqDivisor {
  uint32_t d;   // the divisor, >= 1
  uint32_t m;   // multiplier
  uint32_t l;   // shift, ceil(log2 d)
};

constexpr MxqDivisor mxq_divisor(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && ((uint64_t)1 << l) < d) l++;
  return MxqDivisor{d, (uint32_t)(((((uint64_t)1 << l) - d) << 32) / d + 1), l};
}

constexpr uint32_t mxq_quot(uint32_t n, MxqDivisor v) {
  return (uint32_t)(((((uint64_t)n * v.m) >> 32) + n) >> v.l);
}
