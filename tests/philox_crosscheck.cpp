// Test helper: evaluates Philox4x32-10 with two independent, installed
// source implementations (PyTorch's at::philox_engine and rocRAND's
// philox4x32_10_engine) so the oracle's own Philox can be checked against
// them.  Reads lines "c0 c1 c2 c3 k0 k1" (decimal uint32) from stdin and
// prints "t0 t1 t2 t3 r0 r1 r2 r3" per line.
#include <ATen/core/PhiloxRNGEngine.h>
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdint>
#include <cstdio>

struct RocrandBlock : rocrand_device::philox4x32_10_engine {
  uint4 block(uint4 c, uint2 k) { return ten_rounds(c, k); }
};

int main() {
  unsigned long long c0, c1, c2, c3, k0, k1;
  RocrandBlock rr;
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    // PyTorch: key = seed, counter = (offset lo, offset hi, subsequence lo, subsequence hi).
    uint64_t seed = k0 | (k1 << 32);
    uint64_t subseq = c2 | (c3 << 32);
    uint64_t offset = c0 | (c1 << 32);
    at::philox_engine eng(seed, subseq, offset);
    uint32_t t[4];
    for (int i = 0; i < 4; ++i) t[i] = eng();
    uint4 c = {(unsigned)c0, (unsigned)c1, (unsigned)c2, (unsigned)c3};
    uint2 k = {(unsigned)k0, (unsigned)k1};
    uint4 r = rr.block(c, k);
    std::printf("%u %u %u %u %u %u %u %u\n", t[0], t[1], t[2], t[3], r.x, r.y, r.z, r.w);
  }
  return 0;
}
