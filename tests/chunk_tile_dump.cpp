// Reads lines "c nf nc g" on stdin and prints ssm::chunk_tile(c, nf, nc, g) for each (the
// chunk boundary function the scan kernels and the host plan share), for
// tests/test_chunk_tile.py.  Host code only.
#include <cstdio>
#include "../selective_state_space_02_amd/csrc/launch.hpp"

int main() {
  long long c, nf, nc, g;
  while (std::scanf("%lld %lld %lld %lld", &c, &nf, &nc, &g) == 4)
    std::printf("%lld\n", (long long)ssm::chunk_tile(c, nf, nc, g));
  return 0;
}
