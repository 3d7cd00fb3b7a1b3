// Host check of the statistics passes' work split (pisa_internal.h): the SW ranges partition the
// H * N_b (head, block) pairs into consecutive runs whose lengths differ by at most one,
// stat_owner inverts stat_range_begin, and the partial slots w + h of the (range, head) pairs are
// distinct, below stat_slots, and for each head the run from stat_owner(first pair) + h to
// stat_owner(last pair) + h that the finalize kernel sums. Built with g++ (no GPU).
#define __host__
#define __device__
#include "pisa_internal.h"

#include <cstdio>
#include <set>
#include <vector>

static int fails = 0;
#define CHECK(c, ...)                   \
  do {                                  \
    if (!(c)) {                         \
      if (fails++ < 10) {               \
        std::printf("FAIL: " __VA_ARGS__); \
        std::printf("\n");              \
      }                                 \
    }                                   \
  } while (0)

static void check(int H, int Nb, int SW) {
  pisa::Dims dm{};
  dm.H = H;
  dm.Nb = Nb;
  dm.SW = SW;
  const long long T = (long long)H * Nb;
  CHECK(pisa::stat_range_begin(dm, 0) == 0, "H=%d Nb=%d SW=%d: first range starts at %d", H, Nb, SW,
        pisa::stat_range_begin(dm, 0));
  CHECK(pisa::stat_range_begin(dm, SW) == T, "H=%d Nb=%d SW=%d: last range ends at %d", H, Nb, SW,
        pisa::stat_range_begin(dm, SW));
  const long long lo = T / SW, hi = (T + SW - 1) / SW;
  std::set<int> slots;
  for (int w = 0; w < SW; ++w) {
    const int b = pisa::stat_range_begin(dm, w), e = pisa::stat_range_begin(dm, w + 1);
    CHECK(e - b >= lo && e - b <= hi && e - b >= 1, "H=%d Nb=%d SW=%d: range %d has length %d", H, Nb, SW, w,
          e - b);
    for (int g = b; g < e; ++g) CHECK(pisa::stat_owner(dm, g) == w, "H=%d Nb=%d SW=%d: owner(%d) = %d, not %d", H,
                                      Nb, SW, g, pisa::stat_owner(dm, g), w);
    for (int h = b / Nb; h <= (e - 1) / Nb; ++h) {
      const int slot = w + h;
      CHECK(slots.insert(slot).second, "H=%d Nb=%d SW=%d: slot %d used twice", H, Nb, SW, slot);
      CHECK(slot < pisa::stat_slots(dm), "H=%d Nb=%d SW=%d: slot %d past %d", H, Nb, SW, slot,
            pisa::stat_slots(dm));
    }
  }
  for (int h = 0; h < H; ++h) {  // the slots the finalize kernel sums for head h are those written for h
    std::vector<int> want;
    for (int w = 0; w < SW; ++w) {
      const int b = pisa::stat_range_begin(dm, w), e = pisa::stat_range_begin(dm, w + 1);
      if (b < (h + 1) * Nb && e > h * Nb) want.push_back(w + h);
    }
    const int p0 = pisa::stat_owner(dm, h * Nb) + h, p1 = pisa::stat_owner(dm, h * Nb + Nb - 1) + h;
    CHECK((int)want.size() == p1 - p0 + 1 && want.front() == p0 && want.back() == p1,
          "H=%d Nb=%d SW=%d: head %d sums slots %d..%d", H, Nb, SW, h, p0, p1);
  }
}

int main() {
  for (int H = 1; H <= 9; ++H)
    for (int Nb = 1; Nb <= 40; ++Nb)
      for (int SW = 1; SW <= H * Nb; ++SW) check(H, Nb, SW);
  const int big[][3] = {{40, 591, 512}, {24, 931, 512}, {40, 256, 512}, {24, 72, 432}, {40, 591, 511}, {7, 1, 2}};
  for (const auto& c : big) check(c[0], c[1], c[2]);
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("ranges ok\n");
  return 0;
}
