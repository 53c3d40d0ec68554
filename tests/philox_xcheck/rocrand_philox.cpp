// Prints Philox4x32-10 blocks computed by rocRAND's open-source engine.
// stdin: lines "c0 c1 c2 c3 k0 k1" (hex); stdout: the 4 output words (hex).
// The engine is positioned with key = seed, counter words 2-3 = subsequence and
// counter words 0-1 = offset / 4, so the next four draws are block (c0..c3).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
  unsigned c[4], k[2];
  while (scanf("%x %x %x %x %x %x", &c[0], &c[1], &c[2], &c[3], &k[0], &k[1]) == 6) {
    unsigned long long seed = ((unsigned long long)k[1] << 32) | k[0];
    unsigned long long sub = ((unsigned long long)c[3] << 32) | c[2];
    unsigned long long blk = ((unsigned long long)c[1] << 32) | c[0];
    rocrand_device::philox4x32_10_engine e(seed, sub, 0);
    e.discard(blk * 4ULL);
    unsigned w0 = e(), w1 = e(), w2 = e(), w3 = e();
    printf("%08x %08x %08x %08x\n", w0, w1, w2, w3);
  }
  return 0;
}
