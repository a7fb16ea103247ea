// Prints rocRAND's Philox4x32-10 blocks for counter (position, request, 0, 0) and key = seed.
// Used only as an external reference for the oracle's own Philox: rocRAND's host-side engine is
// run (not copied).  Its counter is (offset/4 low, high, subsequence low, high), so the block for
// counter words (c0, c1, 0, 0) is the engine at subsequence 0 and offset 4 * (c0 + 2^32 c1).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 5) return 2;  // seed first_request n_requests n_positions
  const unsigned long long seed = std::strtoull(argv[1], nullptr, 0);
  const long long req0 = std::atoll(argv[2]);
  const long long n_req = std::atoll(argv[3]);
  const int n_pos = std::atoi(argv[4]);
  for (long long i = req0; i < req0 + n_req; ++i) {
    for (int j = 0; j < n_pos; ++j) {
      const unsigned long long ctr = (unsigned long long)j | ((unsigned long long)i << 32);
      rocrand_device::philox4x32_10_engine e(seed, 0ull, 4ull * ctr);
      const uint4 r = e.next4();
      std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
  }
  return 0;
}
