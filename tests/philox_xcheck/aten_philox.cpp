// Prints Philox4x32-10 blocks computed by ATen's open-source engine (same I/O as
// rocrand_philox.cpp).  ATen's offset counts 128-bit blocks.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>

int main() {
  unsigned c[4], k[2];
  while (scanf("%x %x %x %x %x %x", &c[0], &c[1], &c[2], &c[3], &k[0], &k[1]) == 6) {
    uint64_t seed = ((uint64_t)k[1] << 32) | k[0];
    uint64_t sub = ((uint64_t)c[3] << 32) | c[2];
    uint64_t blk = ((uint64_t)c[1] << 32) | c[0];
    at::Philox4_32 e(seed, sub, blk);
    unsigned w0 = e(), w1 = e(), w2 = e(), w3 = e();
    printf("%08x %08x %08x %08x\n", w0, w1, w2, w3);
  }
  return 0;
}
