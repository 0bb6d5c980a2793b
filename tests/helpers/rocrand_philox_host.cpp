// Host-only helper for the oracle's Philox pin: prints rocRAND's Philox4x32-10 output block for
// (seed, subsequence, offset) triples read from stdin (hex).  rocRAND's engine uses
// key = (seed low, seed high) and counter = (offset / 4 as two words, subsequence as two words),
// so these triples reach any counter whose first two words fit in 62 bits.  No device code runs.
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llx %llx %llx", &seed, &sub, &off) == 3) {
    rocrand_device::philox4x32_10_engine eng(seed, sub, off);
    uint4 r = eng.next4();
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
