// Independent Philox4x32-10 words from rocRAND's open-source engine
// (rocrand/rocrand_philox4x32_10.h), used only to pin the CPU oracle's
// Philox. Host-only build; nothing here is shared with the oracle or the
// GPU library.
//
// stdin : lines "key0 key1 c0 c1 c2 c3" (unsigned 32-bit decimal)
// stdout: lines "w0 w1 w2 w3" = Philox4x32-10(counter, key)
//
// rocRAND's state for (seed, subsequence, offset) has key = (lo(seed),
// hi(seed)), counter words 2..3 = subsequence, and counter words 0..1
// advanced by offset / 4, so skipping 4*n values from a zero counter lands
// on counter (lo(n), hi(n), c2, c3).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned long long k0, k1, c0, c1, c2, c3;
    while (std::scanf("%llu %llu %llu %llu %llu %llu", &k0, &k1, &c0, &c1, &c2, &c3) == 6) {
        const unsigned long long seed = k0 | (k1 << 32);
        const unsigned long long subsequence = c2 | (c3 << 32);
        const unsigned long long n = c0 | (c1 << 32);
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, subsequence, 0ull, &st);
        // add n to the low 64 counter bits in steps that fit skipahead's 64-bit argument
        const unsigned long long low = n & ((1ull << 61) - 1);
        skipahead(4ull * low, &st);
        for (unsigned long long i = 0; i < (n >> 61); ++i) skipahead(1ull << 63, &st);
        unsigned int w[4];
        for (int i = 0; i < 4; ++i) w[i] = rocrand(&st);
        std::printf("%u %u %u %u\n", w[0], w[1], w[2], w[3]);
    }
    return 0;
}
