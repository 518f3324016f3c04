// Host-only reference driver for the oracle's Philox4x32-10 pin.
//
// Reads lines "seed c0 c1 c2 c3" (decimal) on stdin and prints the four
// 32-bit words of rocRAND's philox4x32_10 engine for key = seed and
// counter = (c0, c1, c2, c3).  The engine's (seed, subsequence, offset)
// constructor places the subsequence in counter words 2..3 and offset/4 in
// words 0..1, so the counter is fully addressable.  Runs on the CPU only.
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

int main() {
    unsigned long long seed, c0, c1, c2, c3;
    while (std::scanf("%llu %llu %llu %llu %llu", &seed, &c0, &c1, &c2, &c3) == 5) {
        const unsigned long long sub = (c3 << 32) | c2;
        const unsigned long long ctr01 = (c1 << 32) | c0;
        rocrand_device::philox4x32_10_engine eng(seed, sub, ctr01 * 4ull);
        const uint4 r = eng.next4();
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
