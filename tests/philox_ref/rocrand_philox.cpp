// Test support: prints Philox-4x32-10 output blocks from rocRAND's engine
// (host code, header only), an implementation independent of this
// repository's, to pin the oracle's counter-based generator.
//
//   usage: rocrand_philox SEED ROW J0 COUNT
//   prints COUNT lines "j w0 w1 w2 w3": the block for counter (j, ROW, 0, 0)
//   and key (SEED low 32 bits, SEED high 32 bits), j = J0 .. J0+COUNT-1.
//
// rocRAND's engine starts at counter (0, 0, 0, 0) with that key and steps the
// 128-bit counter once per four outputs; an offset of 4 (j + ROW 2^32)
// outputs therefore lands on counter (j, ROW, 0, 0) (ROW < 2^30, so the
// offset fits in 64 bits).
#include <rocrand/rocrand_kernel.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char **argv) {
  if (argc != 5) return 2;
  const unsigned long long seed = std::strtoull(argv[1], nullptr, 0);
  const unsigned long long row = std::strtoull(argv[2], nullptr, 0);
  const unsigned long long j0 = std::strtoull(argv[3], nullptr, 0);
  const unsigned long long count = std::strtoull(argv[4], nullptr, 0);
  for (unsigned long long j = j0; j < j0 + count; ++j) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, 0, 4ull * (j + (row << 32)), &st);
    const unsigned int w0 = rocrand(&st), w1 = rocrand(&st), w2 = rocrand(&st), w3 = rocrand(&st);
    std::printf("%llu %u %u %u %u\n", j, w0, w1, w2, w3);
  }
  return 0;
}
