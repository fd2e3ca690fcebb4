// Host-side probe: evaluates rocRAND's own Philox4x32-10 block function on
// (counter, key) pairs read from stdin, one "c0 c1 c2 c3 k0 k1" line each (hex),
// and prints the four output words.  Used only to pin the oracle's Philox
// against an implementation it shares nothing with.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

struct Probe : rocrand_device::philox4x32_10_engine {
  uint4 block(uint4 c, uint2 k) { return ten_rounds(c, k); }
};

int main() {
  Probe p;
  unsigned a[6];
  while (std::scanf("%x %x %x %x %x %x", &a[0], &a[1], &a[2], &a[3], &a[4], &a[5]) == 6) {
    uint4 c = {a[0], a[1], a[2], a[3]};
    uint2 k = {a[4], a[5]};
    uint4 o = p.block(c, k);
    std::printf("%08x %08x %08x %08x\n", o.x, o.y, o.z, o.w);
  }
  return 0;
}
