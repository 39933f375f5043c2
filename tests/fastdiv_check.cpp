// Host check of fa::make_fastdiv / fa::fast_div (csrc/fa_internal.h) against the integer
// division they replace in the kernels' work-item decoding: every divisor 1 .. 4096, numerators
// 0 .. 20000, numerators near multiples of the divisor, near 2^31, and pseudo-random ones below
// 2^31.  Prints "ok <count>" or the first mismatch and exits non-zero.
#include <cstdint>
#include <cstdio>

#include "fa_internal.h"

static int check(uint32_t n, uint32_t d, const fa::FastDiv &f, long long *count) {
  ++*count;
  if (fa::fast_div(n, f) != n / d) {
    std::printf("mismatch: n=%u d=%u fast=%u exact=%u\n", n, d, fa::fast_div(n, f), n / d);
    return 1;
  }
  return 0;
}

int main() {
  long long count = 0;
  uint64_t x = 0x9e3779b97f4a7c15ull;  // splitmix64 state
  for (uint32_t d = 1; d <= 4096; ++d) {
    const fa::FastDiv f = fa::make_fastdiv(d);
    for (uint32_t n = 0; n <= 20000; ++n)
      if (check(n, d, f, &count)) return 1;
    for (uint32_t k = 1; k <= 64; ++k) {
      const uint64_t base = (uint64_t)d * (((uint64_t)1 << 31) / d / 64 * k);
      for (int e = -2; e <= 2; ++e) {
        const int64_t n = (int64_t)base + e;
        if (n >= 0 && n < ((int64_t)1 << 31) && check((uint32_t)n, d, f, &count)) return 1;
      }
    }
    for (uint32_t n = 0x7fffffffu - 64; n != 0x80000000u; ++n)
      if (check(n, d, f, &count)) return 1;
    for (int i = 0; i < 2000; ++i) {
      x += 0x9e3779b97f4a7c15ull;
      uint64_t z = x;
      z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
      z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
      z ^= z >> 31;
      if (check((uint32_t)(z & 0x7fffffffu), d, f, &count)) return 1;
    }
  }
  std::printf("ok %lld\n", count);
  return 0;
}
