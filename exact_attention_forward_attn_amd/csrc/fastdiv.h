// Division by a divisor fixed for a whole launch, as one multiply-high and
// two shifts.
//
// A kernel that splits its workgroup id by run-time sizes (query blocks per
// head, heads per batch entry, ...) would otherwise get the compiler's
// general sequence for a division by a kernel argument, which goes through
// the float reciprocal on the vector unit and back to scalar registers: a
// few hundred cycles of dependent instructions at the start of every
// workgroup. The host prepares the constants once per launch instead.
//
// Method: T. Granlund and P. L. Montgomery, "Division by invariant integers
// using multiplication", PLDI 1994, section 4 (unsigned division, N = 32):
// for a divisor 1 <= d < 2^31 let l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1 (it fits 32 bits). Then for every
// 32-bit n, with t = floor(m n / 2^32),
//   floor(n / d) = (t + ((n - t) >> s1)) >> s2,   s1 = min(l, 1), s2 = max(l - 1, 0).
// (n - t cannot underflow: t <= n.)
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__
#else
#define ATTN_HD
#endif

namespace attn {

struct FastDiv {
  uint32_t d;       // the divisor
  uint32_t m;       // the multiplier
  uint32_t s1, s2;  // the two shifts
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d ? d : 1;  // callers never divide by 0; keep the constants defined
  uint32_t l = 0;
  while (l < 32 && (uint64_t(1) << l) < f.d) ++l;
  f.m = (uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - f.d)) / f.d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

ATTN_HD inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
  const uint32_t t = (uint32_t)(((uint64_t)n * f.m) >> 32);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

// quotient and remainder
ATTN_HD inline void fdivmod(uint32_t n, const FastDiv& f, uint32_t& q, uint32_t& r) {
  q = fdiv(n, f);
  r = n - q * f.d;
}

}  // namespace attn
