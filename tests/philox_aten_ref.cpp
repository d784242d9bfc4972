// Prints Philox4x32-10 outputs of PyTorch's ATen engine for counters and keys
// read from stdin (one case per line: c0 c1 c2 c3 k0 k1, decimal). Used only
// by tests/test_oracle_philox.py as an independent library implementation.
// at::philox_engine(seed, subsequence, offset) sets key = (seed lo, seed hi)
// and counter = (offset lo, offset hi, subsequence lo, subsequence hi).
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>

int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    const uint64_t seed = k0 | (k1 << 32);
    const uint64_t subsequence = c2 | (c3 << 32);
    const uint64_t offset = c0 | (c1 << 32);
    at::philox_engine engine(seed, subsequence, offset);
    const uint32_t w0 = engine(), w1 = engine(), w2 = engine(), w3 = engine();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
