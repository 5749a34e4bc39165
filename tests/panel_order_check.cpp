// Host-side check of the panel-pair order used by the pair-symmetric passes
// (PanelOrder in nbody_common.hpp): for many panel counts P, the blocks of
// the launch grid take every pair (I, J), I <= J < P, exactly once; the
// blocks of one XCD (b % 8) take a contiguous stretch of pair numbers in
// ascending order; and within one tile column the pairs are those with
// J in [cS, cS + S).  For column chunks: a chunk's launch takes exactly its
// columns' pairs, every slot of its SlotMap is written once, and the chunk
// reduces add each panel's sums in ascending J over all chunks.  Only host
// code runs (no GPU is needed).
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
    // Column chunks of C panels (C a multiple of the tile side): the blocks of
    // a chunk's launch take exactly the pairs with J in [c0, c1), each once;
    // every slot of the chunk's SlotMap is written by exactly one task side
    // and lies in [0, slots()); and the reduces, chunk after chunk, add each
    // panel's sums for J = 0 .. P-1 once each, in ascending J, in blocks of 32
    // panels that start at multiples of 32.
    for (int C : {32, 64, 96, 128}) {
      std::vector<int> next_j(P, 0);  // the J each panel's running sum expects next
      for (int c0 = 0; c0 < P; c0 += C) {
        const int c1 = P < c0 + C ? P : c0 + C;
        const PanelOrder oc =
            panel_order_range(P, first_pair_of_column(c0), first_pair_of_column(c1));
        const SlotMap map{c0, c1};
        const long long nslots = map.slots();
        std::vector<unsigned char> written((size_t)nslots, 0);
        long long got = 0;
        for (long long b = 0; b < kXcds * oc.per_xcd; ++b) {
          int I, J;
          long long t;
          if (!panel_pair_of_block(oc, b, I, J, t)) continue;
          ++got;
          if (J < c0 || J >= c1 || I > J) {
            std::printf("P=%d C=%d chunk %d: pair (%d, %d) outside the chunk\n", P, C, c0, I, J);
            ++bad;
            continue;
          }
          const long long sides[2] = {map.slot(I, J), I < J ? map.slot(J, I) : -1};
          for (long long sl : sides) {
            if (sl == -1) continue;
            if (sl < 0 || sl >= nslots || written[(size_t)sl]++) {
              std::printf("P=%d C=%d chunk %d: slot %lld of pair (%d, %d) bad or reused\n", P,
                          C, c0, sl, I, J);
              ++bad;
            }
          }
        }
        if (got != first_pair_of_column(c1) - first_pair_of_column(c0)) {
          std::printf("P=%d C=%d chunk %d: %lld pairs taken\n", P, C, c0, got);
          ++bad;
        }
        for (long long sl = 0; sl < nslots; ++sl)
          if (!written[(size_t)sl]) {
            std::printf("P=%d C=%d chunk %d: slot %lld never written\n", P, C, c0, sl);
            ++bad;
            break;
          }
        // the reduce: panels K < c0 add J in [c0, c1), panels in the chunk
        // start afresh and add J in [0, c1); slots of consecutive J adjacent;
        // its blocks of 32 panels start at multiples of 32, as in the whole pass
        for (int K = 0; K < c1; ++K) {
          const int jfirst = K < c0 ? c0 : 0;
          if (jfirst % kPanelTile != 0) {
            std::printf("P=%d C=%d: panel %d block sums start at J=%d\n", P, C, K, jfirst);
            ++bad;
          }
          if (K >= c0 && next_j[K] != 0) {
            std::printf("P=%d C=%d: panel %d starts again at chunk %d\n", P, C, K, c0);
            ++bad;
          }
          if (K < c0 && next_j[K] != c0) {
            std::printf("P=%d C=%d: panel %d expects J=%d at chunk %d\n", P, C, K, next_j[K],
                        c0);
            ++bad;
          }
          for (int J = jfirst; J < c1; ++J)
            if (J > jfirst && map.slot(K, J) != map.slot(K, J - 1) + 1) {
              std::printf("P=%d C=%d: panel %d slots not consecutive at J=%d\n", P, C, K, J);
              ++bad;
              break;
            }
          next_j[K] = c1;
        }
      }
      for (int K = 0; K < P; ++K)
        if (next_j[K] != P) {
          std::printf("P=%d C=%d: panel %d summed up to J=%d only\n", P, C, K, next_j[K]);
          ++bad;
          break;
        }
      if (bad) break;
    }
    // the whole pass is the chunk [0, P): slot K P + J
    const SlotMap whole{0, P};
    if (P > 1 && (whole.slot(P - 1, 1) != (long long)(P - 1) * P + 1 ||
                  whole.slots() != (long long)P * P)) {
      std::printf("P=%d: whole-pass slots are not K P + J\n", P);
      ++bad;
    }
    if (bad) break;
  }
  std::printf("panel order: %zu panel counts, %s\n", sizes.size(), bad ? "FAILED" : "ok");
  return bad ? 1 : 0;
}
