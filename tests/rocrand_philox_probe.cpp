// Host-only probe of rocRAND's open-source Philox4x32-10 engine, used by the oracle's tests as
// an independent library implementation of the Philox block function.  Reads lines
// "c0 c1 c2 c3 k0 k1" (hex) on stdin and prints the four output words of the 10-round block.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

struct block_probe : rocrand_device::philox4x32_10_engine {
    uint4 block(uint4 ctr, uint2 key) { return ten_rounds(ctr, key); }
};

int main() {
    block_probe p;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 out = p.block(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%08x %08x %08x %08x\n", out.x, out.y, out.z, out.w);
    }
    return 0;
}
