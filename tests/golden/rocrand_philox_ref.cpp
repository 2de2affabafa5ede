// Third, independent Philox4x32-10: rocRAND's host-callable engine.
//
// Test helper only.  Reads lines "seed block" (decimal, unsigned 64-bit) from
// stdin and prints the four 32-bit words Philox4x32-10 produces for key =
// (lo32(seed), hi32(seed)) and counter = (lo32(block), hi32(block), 0, 0).
//
// rocRAND's engine keys on the seed the same way and, for subsequence 0,
// skipping 4*block outputs (done in steps) lands its counter on (lo32(block), hi32(block),
// 0, 0); its next four outputs are then the four words of that block.  The
// oracle's own pure-Python generator is checked against this program's output.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
  unsigned long long seed = 0, block = 0;
  while (std::scanf("%llu %llu", &seed, &block) == 2) {
    // Skip to the block in steps small enough that 4*step fits in 64 bits.
    rocrand_device::philox4x32_10_engine eng(seed, 0ULL, 0ULL);
    unsigned long long left = block;
    while (left > 0) {
      unsigned long long step = left < (1ULL << 60) ? left : (1ULL << 60);
      eng.discard(4ULL * step);
      left -= step;
    }
    unsigned int w0 = eng.next();
    unsigned int w1 = eng.next();
    unsigned int w2 = eng.next();
    unsigned int w3 = eng.next();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
