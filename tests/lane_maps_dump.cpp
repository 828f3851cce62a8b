// Prints, as JSON, the lane maps the scan backward's channel reduce-scatter uses (from the
// kernels' own header), for tests/test_lane_maps.py: perm_quarter and perm_xor per lane,
// perm_partial_lane per (t, n, p), chan_partial_lane<V> per (k, p, q).  Host code only.
#include <cstdio>
#include "../selective_state_space_02_amd/csrc/common.hpp"

template <int V>
static void dump_chan(const char* name) {
  constexpr int NP = 16 / V;  // partials per value
  std::printf("\"%s\": [", name);
  bool first = true;
  for (int k = 0; k < V; ++k)
    for (int p = 0; p < NP; ++p)
      for (int q = 0; q < 4; ++q) {
        std::printf("%s[%d, %d, %d, %d]", first ? "" : ", ", k, p, q,
                    ssm::chan_partial_lane<V>(k, p, q));
        first = false;
      }
  std::printf("],\n");
}

int main() {
  std::printf("{\"quarter\": [");
  for (int l = 0; l < 64; ++l) std::printf("%s%d", l ? ", " : "", ssm::perm_quarter(l));
  std::printf("],\n\"xor\": [");
  for (int l = 0; l < 64; ++l) std::printf("%s%d", l ? ", " : "", ssm::perm_xor(l));
  std::printf("],\n\"partial\": [");
  bool first = true;
  for (int t = 0; t < 2; ++t)
    for (int n = 0; n < 16; ++n)
      for (int p = 0; p < 2; ++p) {
        std::printf("%s[%d, %d, %d, %d]", first ? "" : ", ", t, n, p,
                    ssm::perm_partial_lane(t, n, p));
        first = false;
      }
  std::printf("],\n");
  dump_chan<8>("chan8");
  dump_chan<4>("chan4");
  dump_chan<2>("chan2");
  std::printf("\"end\": 0}\n");
  return 0;
}
