// Test-only helper: evaluates rocRAND's Philox4x32-10 engine (ROCm headers,
// compiled for the host) on arbitrary (counter, key) records, so that a CPU
// test can compare the oracle's own numpy Philox against an independent
// implementation.  Neither the oracle nor the HIP library uses this file.
//
// stdin : records of six little-endian uint32 (c0, c1, c2, c3, k0, k1)
// stdout: records of four uint32 (x0, x1, x2, x3)
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdint>
#include <cstdio>
#include <vector>

int main() {
  std::vector<uint32_t> rec(6);
  while (std::fread(rec.data(), sizeof(uint32_t), 6, stdin) == 6) {
    const unsigned long long seed = (unsigned long long)rec[4] | ((unsigned long long)rec[5] << 32);
    const unsigned long long subsequence = (unsigned long long)rec[2] | ((unsigned long long)rec[3] << 32);
    // Counter words z, w come from the subsequence; x, y from the offset
    // (four outputs per counter).  Word y is added in chunks below 2^30 so
    // that the offset never overflows 64 bits.
    rocrand_device::philox4x32_10_engine e(seed, subsequence, 4ull * rec[0]);
    unsigned long long c1 = rec[1];
    while (c1) {
      const unsigned long long part = c1 < (1ull << 29) ? c1 : (1ull << 29);
      e.discard(part << 34);
      c1 -= part;
    }
    const uint4 r = e.next4();
    const uint32_t o[4] = {r.x, r.y, r.z, r.w};
    std::fwrite(o, sizeof(uint32_t), 4, stdout);
  }
  return 0;
}
