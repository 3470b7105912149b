// Host check of the kernels' packed keep compare (fa2::keep_lt_word in
// csrc/common.hpp, compiled here for the host only): for every threshold
// 0 .. 256, every byte position of a 32-bit generator word and every byte value,
// bit 8 b + 7 of the result equals the plain comparison value < threshold, the
// other bits are zero, and the other three bytes come from a fixed LCG. Prints
// the number of mismatches and exits nonzero if there is one.
#include <cstdio>

#include "common.hpp"

int main() {
  unsigned bad = 0, state = 12345u;
  auto next = [&]() {
    state = state * 1664525u + 1013904223u;
    return state;
  };
  for (unsigned t = 0; t <= 256; ++t) {
    for (int byte = 0; byte < 4; ++byte) {
      for (unsigned b = 0; b < 256; ++b) {
        const uint32_t x = (next() & ~(0xFFu << (8 * byte))) | (b << (8 * byte));
        const uint32_t m = fa2::keep_lt_word(x, t);
        if ((m & ~0x80808080u) != 0u) ++bad;
        if (((m >> (8 * byte + 7)) & 1u) != (b < t ? 1u : 0u)) ++bad;
      }
    }
  }
  printf("%u mismatch(es)\n", bad);
  return bad != 0;
}
