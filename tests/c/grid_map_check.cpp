// Host check of the kernels' workgroup-to-(head, block) map (fa2::grid_map in
// csrc/common.hpp, compiled here for the host only): for every head group size
// the kernels use or might use (1, 2, 4, 8), both head orders, both block
// orders and a range of head and block counts (multiples of 8, 16 and 32 among
// them, so every branch is taken), the ids 0 .. bh_count * nblk - 1 cover each
// (head, block) pair exactly once and stay in range. Prints the number of
// failures and exits nonzero if there is one.
#include <cstdio>
#include <vector>

#include "common.hpp"

static unsigned failures = 0;

template <int G, bool NEIGHBOURS>
static void check(int nblk, int bh_count, bool descending) {
  std::vector<unsigned char> seen((size_t)nblk * bh_count, 0);
  for (int id = 0; id < nblk * bh_count; ++id) {
    int bh = -1, blk = -1;
    fa2::grid_map<G, NEIGHBOURS>(id, nblk, bh_count, descending, bh, blk);
    if (bh < 0 || bh >= bh_count || blk < 0 || blk >= nblk) {
      ++failures;
      continue;
    }
    if (seen[(size_t)bh * nblk + blk]++) ++failures;
  }
}

template <int G>
static void check_all(int nblk, int bh_count) {
  for (int desc = 0; desc < 2; ++desc) {
    check<G, false>(nblk, bh_count, desc != 0);
    check<G, true>(nblk, bh_count, desc != 0);
  }
}

int main() {
  const int blocks[] = {1, 2, 3, 5, 32, 64, 65};
  for (int nblk : blocks) {
    for (int bh = 1; bh <= 72; ++bh) {
      check_all<1>(nblk, bh);
      check_all<2>(nblk, bh);
      check_all<4>(nblk, bh);
      check_all<8>(nblk, bh);
    }
    for (int bh : {96, 128, 256, 384}) {
      check_all<1>(nblk, bh);
      check_all<2>(nblk, bh);
      check_all<4>(nblk, bh);
      check_all<8>(nblk, bh);
    }
  }
  printf("%u failure(s)\n", failures);
  return failures != 0;
}
