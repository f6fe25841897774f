// The host codec's length limiter (boundary package-merge, df11_host.cpp)
// against the oracle's package-merge (oracle/df11_oracle.c) at every limit
// from the smallest feasible one upwards, on seeded histograms: uniform
// small counts, Fibonacci runs (the deepest Huffman trees), powers of two and
// near-ties.  Both take a leaf before a package of equal weight and order
// leaves by (count, symbol), so the length vectors must be equal, not only
// their cost.  Test infrastructure: built by tests/test_sanitize.py with
// AddressSanitizer and UndefinedBehaviorSanitizer; it includes the codec's
// source to reach the limiter, which the library does not export.  Prints
// "limiter ok" at the end.
#include "../../entropy_decoding_amd/csrc/df11_host.cpp"

#include <cstdio>
#include <random>

extern "C" int oracle_limited_lengths(const uint64_t *counts, int limit, uint8_t *lens);

int main() {
    std::mt19937_64 rng(2024);
    long bad = 0, trials = 0;
    for (int it = 0; it < 12000; it++) {
        uint64_t c[kSyms] = {};
        const int n = 2 + int(rng() % (it % 2 ? 40 : 255));
        std::vector<int> order(kSyms);
        for (int s = 0; s < kSyms; s++) order[s] = s;
        std::shuffle(order.begin(), order.end(), rng);
        const int mode = int(rng() % 4);
        uint64_t fa = 1, fb = 1;
        for (int i = 0; i < n; i++) {
            uint64_t v;
            if (mode == 0) {
                v = 1 + rng() % 100;
            } else if (mode == 1) {
                v = fa;
                const uint64_t t = fa + fb;
                fa = fb;
                fb = t > (uint64_t(1) << 50) ? 1 : t;
                if (fb == 1) fa = 1;
            } else if (mode == 2) {
                v = uint64_t(1) << (rng() % 40);
            } else {
                v = 1 + rng() % 3;
            }
            c[order[i]] = v;
        }
        int least = 0;
        while ((1 << least) < n) least++;
        for (int limit = least; limit <= std::min(32, least + 5); limit++) {
            uint8_t a[kSyms], b[kSyms];
            const int ma = package_merge(c, limit, a);
            const int mb = oracle_limited_lengths(c, limit, b);
            trials++;
            if (ma != mb || ma > limit || std::memcmp(a, b, kSyms) != 0) {
                if (bad < 5) std::printf("mismatch: trial %d, %d symbols, limit %d\n", it, n, limit);
                bad++;
            }
        }
    }
    std::printf("%ld limits checked, %ld mismatches\n", trials, bad);
    if (bad) return 1;
    std::printf("limiter ok\n");
    return 0;
}
