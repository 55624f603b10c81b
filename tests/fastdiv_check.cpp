// Host-side check of swrt::FastDiv (the multiply-shift divider the kernels
// use for word -> row -> prefix decomposition): compares it with integer
// division over edge numerators and pseudo-random ones for many divisors.
#include "../sliding_window_ring_tensor_amd/csrc/swrt_device.hpp"

#include <cstdio>

int main() {
  uint64_t x = 0x9E3779B97F4A7C15ull, bad = 0, n_checks = 0;
  auto next = [&x]() { x ^= x << 13; x ^= x >> 7; x ^= x << 17; return x; };
  auto check = [&](uint32_t d, uint32_t n) {
    const swrt::FastDiv f(d);
    ++n_checks;
    if (f.div(n) != n / d) {
      if (bad++ < 10) std::printf("FastDiv(%u).div(%u) = %u, want %u\n", d, n, f.div(n), n / d);
    }
  };
  const uint32_t top = 0x7FFFFFFFu;
  for (uint32_t d = 1; d <= 4096; ++d) {
    for (uint32_t n : {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, top, top - 1, top - d})
      check(d, n);
    for (int k = 0; k < 200; ++k) check(d, uint32_t(next() & top));
  }
  for (int k = 0; k < 200000; ++k) {
    const uint32_t d = uint32_t(next() % top) + 1;
    const uint32_t q = uint32_t(next() % (top / d + 1));
    check(d, uint32_t(next() & top));
    const uint64_t m = uint64_t(q) * d;
    if (m <= top) { check(d, uint32_t(m)); if (m) check(d, uint32_t(m - 1)); }
  }
  for (uint32_t s = 0; s < 31; ++s) check(1u << s, top), check((1u << s) + 1, top);
  std::printf("%llu checks, %llu wrong\n", (unsigned long long)n_checks, (unsigned long long)bad);
  return bad ? 1 : 0;
}
