// Test support: prints rocRAND's Philox4x32-10 block function for counters and
// keys read from stdin, one case per line: "c0 c1 c2 c3 k0 k1" (hex) ->
// "r0 r1 r2 r3" (hex).  rocRAND is an independent implementation of the
// generator of Salmon et al. (SC'11); the test suite uses it to pin the CPU
// oracle's own Philox.  Host code only: no GPU is touched.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

struct philox_block : rocrand_device::philox4x32_10_engine {
    uint4 run(uint4 counter, uint2 key) { return ten_rounds(counter, key); }
};

int main()
{
    philox_block gen;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = gen.run(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
