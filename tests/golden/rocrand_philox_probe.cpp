// Cross-check helper: prints Philox4x32-10 blocks computed by rocRAND's
// header-only engine (host side), for counters/keys read from stdin as
// "c0 c1 c2 c3 k0 k1" lines. Used only by the oracle's CPU tests.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

struct Block : rocrand_device::philox4x32_10_engine {
    uint4 at(uint4 c, uint2 k) { return this->ten_rounds(c, k); }
};

int main() {
    Block b;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = b.at(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
