// Independent Philox4x32-10 reference for the oracle's generator: rocRAND's engine,
// used only through its public host/device API (rocrand_init / rocrand), run on the CPU.
// rocRAND's documented mapping: the seed is the key, a subsequence is 2^66 numbers
// (the high 64 bits of the counter), and the offset skips single 32-bit outputs.
// stdin: lines "seed subsequence offset"; stdout: four consecutive outputs per line.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, sub, off, &st);
    unsigned int a = rocrand(&st), b = rocrand(&st), c = rocrand(&st), d = rocrand(&st);
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
