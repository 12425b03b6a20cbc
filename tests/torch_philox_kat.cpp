// Known-answer source for the oracle's Philox4x32-10: PyTorch's header-only
// at::philox_engine, an implementation written independently of the oracle.
// Reads "seed subsequence offset" triples from stdin and prints the four
// 32-bit words of the block at that (seed, subsequence, offset).
#include <ATen/core/PhiloxRNGEngine.h>
#include <cinttypes>
#include <cstdio>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    at::philox_engine eng(seed, sub, off);
    uint32_t w0 = eng(), w1 = eng(), w2 = eng(), w3 = eng();
    std::printf("%" PRIu32 " %" PRIu32 " %" PRIu32 " %" PRIu32 "\n", w0, w1, w2, w3);
  }
  return 0;
}
