// Host-only helper for the oracle's Philox pin: prints Philox4x32-10 output
// words computed by rocRAND's engine for (counter, key) quadruples read from
// stdin. rocRAND's engine keys on the 64-bit seed and puts the 64-bit
// subsequence in counter words 2..3 and offset/4 in counter words 0..1.
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdint>

int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    const unsigned long long seed = k0 | (k1 << 32);
    const unsigned long long subsequence = c2 | (c3 << 32);
    rocrand_device::philox4x32_10_engine e(seed, subsequence, 0);
    // counter words 0..1 hold a 64-bit block index; skip that many 4-word blocks
    const unsigned long long block = c0 | (c1 << 32);
    e.discard(block * 4ull);
    unsigned w0 = e(), w1 = e(), w2 = e(), w3 = e();
    std::printf("%u %u %u %u\n", w0, w1, w2, w3);
  }
  return 0;
}
