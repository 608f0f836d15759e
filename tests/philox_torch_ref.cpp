// Prints word 0..3 of Philox4x32-10 as computed by PyTorch's header-only
// at::philox_engine (an independent open-source implementation of the same
// published generator).  Reads lines "c0 c1 c2 c3 k0 k1" (hex) from stdin.
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>
int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint64_t seed = ((uint64_t)k1 << 32) | k0;
    uint64_t subseq = ((uint64_t)c3 << 32) | c2;
    uint64_t offset = ((uint64_t)c1 << 32) | c0;
    at::philox_engine e(seed, subseq, offset);
    unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%08x %08x %08x %08x\n", a, b, c, d);
  }
  return 0;
}
