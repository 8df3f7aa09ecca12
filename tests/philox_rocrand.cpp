// Host-side reference for the Philox4x32-10 pin of the dropout oracle:
// rocRAND's header-only philox4x32_10 engine, compiled for the CPU.
// Reads lines "c0 c1 c2 c3 k0 k1" (decimal 32-bit words) from stdin and
// prints the four 32-bit output words of the block with counter
// (c0, c1, c2, c3) and key (k0, k1).
//
// rocRAND addresses a block through (seed, subsequence, offset): the key is
// the seed's low and high words, the subsequence sets counter words 2 and 3,
// and every 4 numbers of offset advance counter words 0 and 1 by one (the
// offset is a 64-bit number count, so the 64-bit block count of words 0 and 1
// is skipped in steps small enough for it).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
  unsigned long long c[4], k[2];
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c[0], &c[1], &c[2], &c[3], &k[0], &k[1]) ==
         6) {
    const unsigned long long seed = (k[1] << 32) | k[0];
    const unsigned long long subsequence = (c[3] << 32) | c[2];
    rocrand_device::philox4x32_10_engine e(seed, subsequence, 0);
    for (unsigned long long left = (c[1] << 32) | c[0]; left > 0;) {
      const unsigned long long step = left < (1ull << 60) ? left : (1ull << 60);
      e.discard(4 * step);
      left -= step;
    }
    const uint4 r = e.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
