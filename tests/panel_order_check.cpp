// Host-side check of the panel-pair order used by the pair-symmetric passes
// (PanelOrder in nbody_common.hpp): for many panel counts P, the blocks of
// the launch grid take every pair (I, J), I <= J < P, exactly once; the
// blocks of one XCD (b % 8) take a contiguous stretch of pair numbers in
// ascending order; and within one tile column the pairs are those with
// J in [cS, cS + S).  Only host code runs (no GPU is needed).
#include <cstdio>
#include <vector>

#include "nbody_common.hpp"

int main() {
  using namespace nbody;
  int bad = 0;
  std::vector<int> sizes;
  for (int P = 1; P <= 130; ++P) sizes.push_back(P);
  for (int P : {255, 256, 257, 489, 511, 512, 513, 1000, 2049}) sizes.push_back(P);
  for (int P : sizes) {
    const PanelOrder o = panel_order(P);
    const long long blocks = kXcds * o.per_xcd;
    std::vector<unsigned char> seen((size_t)P * P, 0);
    std::vector<long long> last(kXcds, -1);
    long long taken = 0;
    for (long long b = 0; b < blocks; ++b) {
      int I, J;
      long long t;
      if (!panel_pair_of_block(o, b, I, J, t)) continue;
      ++taken;
      if (I < 0 || J < 0 || I > J || J >= P) {
        std::printf("P=%d block %lld: bad pair (%d, %d)\n", P, b, I, J);
        ++bad;
        continue;
      }
      if (seen[(size_t)I * P + J]++) {
        std::printf("P=%d: pair (%d, %d) taken twice\n", P, I, J);
        ++bad;
      }
      const int x = (int)(b % kXcds);
      if (last[x] >= 0 && t != last[x] + 1) {
        std::printf("P=%d: XCD %d jumps from %lld to %lld\n", P, x, last[x], t);
        ++bad;
      }
      last[x] = t;
      // tile column of t holds exactly the pairs with J in [cS, cS + S)
      const long long c = J / o.S;
      const long long lo = (o.S * c) * (o.S * c + 1) / 2;
      const long long hi = (o.S * (c + 1)) * (o.S * (c + 1) + 1) / 2;
      if (t < lo || t >= hi) {
        std::printf("P=%d: pair (%d, %d) numbered %lld outside its tile column\n", P, I, J, t);
        ++bad;
      }
    }
    if (taken != o.pairs) {
      std::printf("P=%d: %lld pairs taken, %lld expected\n", P, taken, o.pairs);
      ++bad;
    }
    if (bad) break;
  }
  std::printf("panel order: %zu panel counts, %s\n", sizes.size(), bad ? "FAILED" : "ok");
  return bad ? 1 : 0;
}
