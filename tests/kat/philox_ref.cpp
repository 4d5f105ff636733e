// Host-side reference outputs of Philox4x32-10 from two independent
// open-source implementations (ATen's PhiloxRNGEngine.h and rocRAND's
// rocrand_philox4x32_10.h), used only to pin the oracle's generator.
// Reads lines "c0 c1 c2 c3 k0 k1" (decimal u32) from stdin and prints, per
// line, "aten x0 x1 x2 x3" and, when c1 < 2^30, "rocrand x0 x1 x2 x3".
#include <cstdint>
#include <cstdio>
#include <ATen/core/PhiloxRNGEngine.h>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
  unsigned long long c[4], k[2];
  while (std::scanf("%llu %llu %llu %llu %llu %llu", &c[0], &c[1], &c[2], &c[3],
                    &k[0], &k[1]) == 6) {
    const uint64_t seed = k[0] | (k[1] << 32);
    const uint64_t subseq = c[2] | (c[3] << 32);
    const uint64_t offset = c[0] | (c[1] << 32);
    at::philox_engine a(seed, subseq, offset);
    uint32_t o0 = a(), o1 = a(), o2 = a(), o3 = a();
    std::printf("aten %u %u %u %u\n", o0, o1, o2, o3);
    if (c[1] < (1ull << 30)) {
      rocrand_device::philox4x32_10_engine r(seed, subseq, offset * 4ull);
      uint32_t q0 = r(), q1 = r(), q2 = r(), q3 = r();
      std::printf("rocrand %u %u %u %u\n", q0, q1, q2, q3);
    } else {
      std::printf("rocrand skip\n");
    }
  }
  return 0;
}
