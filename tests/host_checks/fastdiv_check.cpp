// Host check of the launch-time division used by the vector kernel's index
// math (rope_fastdiv.hpp): exhaustive for small divisors and dividends,
// random and boundary cases up to 2^31. Built with g++ by tests/test_host_logic.py.
#include "rope_fastdiv.hpp"
#include <cstdio>
#include <random>
int main() {
  std::mt19937_64 g(1);
  long bad = 0, n_checked = 0;
  for (uint32_t d = 1; d < 5000; ++d) { auto f = rope::make_fastdiv(d); for (uint32_t n = 0; n < 70000; ++n) { if (rope::fast_div(n, f) != n / d) ++bad; ++n_checked; } }
  for (int t = 0; t < 2000000; ++t) { uint32_t d = 1 + (uint32_t)(g() % ((1u<<31) - 1)); uint32_t n = (uint32_t)(g() % (1u<<31)); auto f = rope::make_fastdiv(d); if (rope::fast_div(n, f) != n / d) ++bad; ++n_checked;
    uint32_t n2 = (n / d) * d; if (rope::fast_div(n2, f) != n2 / d) ++bad; if (n2 && rope::fast_div(n2 - 1, f) != (n2 - 1) / d) ++bad; n_checked += 2; }
  for (uint32_t d : {1u, 2u, 3u, 7u, 8u, 12u, 16u, 4096u, 8192u, 65535u, (1u<<31)-1u, 1u<<30}) { auto f = rope::make_fastdiv(d); for (uint32_t n : {0u, 1u, d-1, d, d+1, (1u<<31)-1u, (1u<<31)-2u}) { if (n >= (1u<<31)) continue; if (rope::fast_div(n, f) != n / d) ++bad; ++n_checked; } }
  printf("checked %ld, bad %ld\n", n_checked, bad);
  return bad != 0;
}
