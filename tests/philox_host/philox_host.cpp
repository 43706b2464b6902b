// Host-side check of the library's dropout generator (fa_philox.h), built
// for the CPU: the same header the kernels include, instantiated on the host.
// Reads lines "c0 c1 c2 c3 k0 k1" (decimal) from stdin and prints the four
// Philox4x64-10 output words of each in hex. With argument "mul" it instead
// checks mulhilo64 against the compiler's 128-bit product on many pairs and
// prints "ok" or the first mismatch.
#include <cstdint>
#include <cstdio>
#include <random>
#include <cstring>

#include "fa_philox.h"

int main(int argc, char** argv) {
  if (argc > 1 && !strcmp(argv[1], "mul")) {
    std::mt19937_64 g(20261203);
    for (int i = 0; i < 1000000; ++i) {
      uint64_t a = g(), b = g();
      if (i % 7 == 0) a = ~0ull;
      if (i % 11 == 0) b = ~0ull;
      if (i % 13 == 0) a >>= 32;
      uint64_t hi;
      const uint64_t lo = fa::mulhilo64(a, b, &hi);
      const unsigned __int128 p = (unsigned __int128)a * b;
      if (lo != (uint64_t)p || hi != (uint64_t)(p >> 64)) {
        printf("mismatch %llu %llu\n", (unsigned long long)a, (unsigned long long)b);
        return 1;
      }
    }
    printf("ok\n");
    return 0;
  }
  unsigned long long c[4], k[2];
  while (scanf("%llu %llu %llu %llu %llu %llu", &c[0], &c[1], &c[2], &c[3], &k[0], &k[1]) == 6) {
    uint64_t w[4] = {c[0], c[1], c[2], c[3]};
    fa::philox4x64_10(w, k[0], k[1]);
    printf("%016llx %016llx %016llx %016llx\n", (unsigned long long)w[0],
           (unsigned long long)w[1], (unsigned long long)w[2], (unsigned long long)w[3]);
  }
  return 0;
}
