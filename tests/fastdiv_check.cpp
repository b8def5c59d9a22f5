// Checks the launch-time division constants (csrc/fastdiv.h) against the
// hardware division: every n, d < 3000, random 32-bit n over random and
// small divisors, and the edges of the 32-bit range. Prints OK and exits 0
// when every quotient and remainder match.
#include "fastdiv.h"
#include <cstdio>
#include <random>
using namespace attn;
int main() {
  std::mt19937_64 g(1);
  long bad = 0, n_checks = 0;
  auto check = [&](uint32_t n, uint32_t d) {
    FastDiv f = make_fastdiv(d);
    uint32_t q, r; fdivmod(n, f, q, r);
    ++n_checks;
    if (q != n / d || r != n % d) { if (bad < 5) printf("bad n=%u d=%u q=%u\n", n, d, q); ++bad; }
  };
  for (uint32_t d = 1; d < 3000; ++d) for (uint32_t n = 0; n < 3000; ++n) check(n, d);
  for (int i = 0; i < 2000000; ++i) { uint32_t d = (uint32_t)(g() % 0x7fffffffu) + 1; uint32_t n = (uint32_t)g(); check(n, d); }
  for (int i = 0; i < 2000000; ++i) { uint32_t d = (uint32_t)(g() % 1000) + 1; uint32_t n = (uint32_t)g(); check(n, d); }
  for (uint32_t d : {1u, 2u, 3u, 7u, 64u, 0x7fffffffu, 0x40000000u, 0x40000001u})
    for (uint32_t n : {0u, 1u, d - 1, d, d + 1, 0x7fffffffu, 0x80000000u, 0xfffffffeu, 0xffffffffu}) check(n, d);
  printf("%s %ld checks\n", bad ? "FAIL" : "OK", n_checks);
  return bad != 0;
}
