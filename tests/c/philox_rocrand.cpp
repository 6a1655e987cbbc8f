// Philox4x32-10 blocks from ROCm's rocRAND library, on the host, as an
// independent check of the oracle's generator (test infrastructure only).
//
// rocRAND's philox4x32_10_engine keeps its ten-round block function
// protected; a derived class calls it directly, so any counter and key can
// be evaluated (the engine's own seed/offset interface only reaches
// counters in its stream order).
//
// stdin: one case per line, six hex words "c0 c1 c2 c3 k0 k1" (word 0 first)
// stdout: one line per case, the four output words in hex.
// Built host-only (no device code): hipcc -x hip --offload-host-only.
#include <cstdio>

#include <rocrand/rocrand_philox4x32_10.h>

namespace {
struct Block : rocrand_device::philox4x32_10_engine {
    uint4 eval(uint4 counter, uint2 key) { return ten_rounds(counter, key); }
};
}  // namespace

int main() {
    Block block;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        const uint4 r = block.eval(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
