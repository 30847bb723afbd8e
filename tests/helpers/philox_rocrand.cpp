// Prints Philox-4x32-10 blocks computed by rocRAND's own engine, for
// counters and keys read from stdin (one "c0 c1 c2 c3 k0 k1" line each).
// rocRAND is an independent implementation of the published generator; the
// test suite compares the oracle's Philox with it.
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    unsigned long long seed = (unsigned long long)k0 | ((unsigned long long)k1 << 32);
    unsigned long long subsequence = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
    unsigned long long block = (unsigned long long)c0 | ((unsigned long long)c1 << 32);
    // counter = (block, subsequence) when the offset is 4 * block numbers
    rocrand_device::philox4x32_10_engine e(seed, subsequence, 4ull * block);
    uint4 r = e.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
