// Host-side probe: evaluates rocRAND's Philox4x32-10 block function (an independent
// implementation of the SC'11 generator) on counter/key words read from stdin, one
// "c0 c1 c2 c3 k0 k1" line per block, and prints the four output words.
// Used only by the CPU test suite as a library cross-check of the oracle's Philox.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

struct PhiloxBlock : rocrand_device::philox4x32_10_engine {
    uint4 block(uint4 c, uint2 k) { return ten_rounds(c, k); }
};

int main() {
    PhiloxBlock eng;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = eng.block(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
