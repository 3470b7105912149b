// Reference Philox4x32-10 blocks from rocRAND's engine (rocrand_philox4x32_10.h,
// host-callable), for pinning the oracle's generator: each input line
// "c0 c1 c2 c3 k0 k1" (hexadecimal 32-bit words) gives one output line with the
// four 32-bit words of the block, in hexadecimal.
#include <cstdio>

#include <rocrand/rocrand_philox4x32_10.h>

struct Engine : rocrand_device::philox4x32_10_engine {
  uint4 block(uint4 counter, uint2 key) { return ten_rounds(counter, key); }
};

int main() {
  Engine e;
  unsigned c0, c1, c2, c3, k0, k1;
  while (scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    const uint4 r = e.block(uint4{c0, c1, c2, c3}, uint2{k0, k1});
    printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
