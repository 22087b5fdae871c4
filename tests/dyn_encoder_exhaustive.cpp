// Host program run by tests/test_host_lib.py: the dynamic-code encoder the kernels
// use (a guess from the code's construction plus a one-step check) must give the
// same code as a plain binary search over the midpoint table for every float in
// [0, 1], for the signed (7 magnitude bits) and unsigned (8 bits) codes.
// Prints the mismatch count; exit status 0 when there are none.
#include <cstdio>
#include <thread>
#include <vector>

#include "../optimizer_gemm_amd/csrc/forge_internal.h"

int main() {
  static constexpr forge::DynTables t = forge::make_dyn_tables();
  const uint32_t last = 0x3F800000u;  // bits of 1.0f
  const unsigned nt = 8;
  std::vector<long> bad(nt, 0);
  std::vector<std::thread> th;
  for (unsigned w = 0; w < nt; ++w)
    th.emplace_back([&, w] {
      for (uint64_t u = w; u <= last; u += nt) {
        float a;
        const uint32_t b = (uint32_t)u;
        memcpy(&a, &b, 4);
        bad[w] += forge::dyn_search_fast<7>(t.ms, a) != forge::dyn_search<128>(t.ms, a);
        bad[w] += forge::dyn_search_fast<8>(t.mu, a) != forge::dyn_search<256>(t.mu, a);
      }
    });
  long total = 0;
  for (unsigned w = 0; w < nt; ++w) {
    th[w].join();
    total += bad[w];
  }
  printf("%ld mismatches over %u floats\n", total, last + 1);
  return total ? 1 : 0;
}
