// Unsigned division by a run-time constant d >= 1 with a precomputed
// multiplier (round-up method of Granlund and Montgomery, "Division by
// Invariant Integers using Multiplication", 1994): for n < 2^32,
// n / d == (umulhi(n, m) + n) >> s with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1.  Plain C++ (no HIP), so the host
// constants can be built and checked by an ordinary compiler.
#pragma once

#include <stdint.h>

namespace kvq {

struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}

// The quotient the device code computes from the constants (its umulhi is the
// high word of the 64-bit product).
inline uint32_t fastdiv_host(uint32_t n, const FastDiv& f) {
  const uint64_t hi = ((uint64_t)n * f.m) >> 32;
  return (uint32_t)((hi + n) >> f.s);
}

}  // namespace kvq
