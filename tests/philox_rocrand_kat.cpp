// Host-only helper for the oracle's Philox pin: reads lines
// "c0 c1 c2 c3 k0 k1" (decimal 32-bit words, c1 < 2^30) from stdin and prints
// the four output words of rocRAND's open-source Philox4x32-10 engine for
// that counter and key.  The engine's key is its 64-bit seed, counter words
// 2-3 are its subsequence, and counter words 0-1 advance with its offset in
// blocks of four numbers.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    const unsigned long long seed = (k1 << 32) | k0;
    const unsigned long long sub = (c3 << 32) | c2;
    const unsigned long long blk = (c1 << 32) | c0;
    rocrand_device::philox4x32_10_engine eng(seed, sub, 0);
    eng.discard(blk * 4ULL);
    const uint4 r = eng.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
