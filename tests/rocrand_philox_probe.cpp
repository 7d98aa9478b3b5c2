// Host-only probe: prints the four Philox4x32-10 words that ROCm's rocRAND host/device
// header produces for each (seed, counter) line on stdin.  Used by a CPU test as an
// external pin of the oracle's generator; never linked into the oracle or the library.
// Input lines: seed c0 c1 c2 c3 (decimal).  c1 must be < 2^30 so that the offset
// 4 * (c0 | c1 << 32) below does not overflow 64 bits.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
    unsigned long long seed, c0, c1, c2, c3;
    while (std::scanf("%llu %llu %llu %llu %llu", &seed, &c0, &c1, &c2, &c3) == 5) {
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, c2 | (c3 << 32), 4ull * (c0 | (c1 << 32)), &st);
        unsigned a = rocrand(&st), b = rocrand(&st), c = rocrand(&st), d = rocrand(&st);
        std::printf("%u %u %u %u\n", a, b, c, d);
    }
    return 0;
}
