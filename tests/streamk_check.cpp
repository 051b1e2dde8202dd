// streamk_check.cpp -- host-side checks of the stream-K share arithmetic in
// dense_gemm_06_amd/csrc/streamk.h (built by tests/test_streamk_host.py with hipcc,
// host code only): the corrected double-precision quotient against exact integer
// division, and the share bounds, pieces and owner search against a plain integer
// restatement, over every tail size and share count of small grids and random large
// arguments. Prints "0 failures" when everything agrees.
#include <stdint.h>
#include <stdio.h>

#include <random>

#include "../dense_gemm_06_amd/csrc/streamk.h"

static int fails = 0;
#define CHECK(c, ...)                        \
    do {                                     \
        if (!(c)) {                          \
            if (fails < 20) printf(__VA_ARGS__); \
            ++fails;                         \
        }                                    \
    } while (0)

static int64_t bound_ref(int w, int G, int64_t iters, int KT) {
    int64_t b = (int64_t)w * iters / G;
    const int64_t r = b % KT;
    if (r != 0) {
        if (r < 4) b -= r;
        else if (KT - r < 4) b += KT - r;
    }
    return b;
}

int main() {
    std::mt19937_64 rng(7);
    // quotients: random and adversarial (a = q * d - 1, q * d, q * d + 1)
    for (int i = 0; i < 2000000; ++i) {
        const int64_t d = (int64_t)(rng() % ((1ull << 31) - 1)) + 1;
        const int64_t a = (int64_t)(rng() % (1ull << 53));
        CHECK(dg::sk_div(a, d) == a / d, "sk_div(%lld, %lld)\n", (long long)a, (long long)d);
        const int64_t q = (int64_t)(rng() % ((1ull << 53) / (uint64_t)d));
        for (int64_t e = -1; e <= 1; ++e) {
            const int64_t x = q * d + e;
            if (x >= 0 && x < (1ll << 53)) CHECK(dg::sk_div(x, d) == x / d, "sk_div(%lld, %lld)\n", (long long)x, (long long)d);
        }
    }
    // bounds, pieces and owners
    for (int KT = 8; KT <= 70; KT += 3)
        for (int G = 2; G <= 40; ++G)
            for (int S = 1; S < G; ++S) {
                const int64_t iters = (int64_t)S * KT;
                if (iters / G < 4) continue;
                for (int w = 0; w <= G; ++w)
                    CHECK(dg::sk_bound(w, G, iters, KT) == bound_ref(w, G, iters, KT), "bound %d %d %d %d\n", w, G, S, KT);
                for (int64_t it = 0; it < iters; ++it) {
                    const int o = dg::sk_owner(it, G, iters, KT);
                    CHECK(dg::sk_bound(o, G, iters, KT) <= it && (o == G - 1 || dg::sk_bound(o + 1, G, iters, KT) > it),
                          "owner %lld %d %d %d\n", (long long)it, G, S, KT);
                }
                for (int w = 0; w < G; ++w) {
                    const int64_t b0 = bound_ref(w, G, iters, KT), b1 = bound_ref(w + 1, G, iters, KT);
                    int64_t covered = 0;
                    for (int p = 0; p < 2; ++p) {
                        int t, kb, nk;
                        if (!dg::sk_piece(w, p, G, S, KT, t, kb, nk)) continue;
                        const int64_t s = (int64_t)t * KT + kb;
                        CHECK(s >= b0 && s + nk <= b1 && nk >= 4 && kb + nk <= KT, "piece %d %d %d %d %d\n", w, p, G, S, KT);
                        covered += nk;
                    }
                    CHECK(covered == b1 - b0, "cover %d %d %d %d\n", w, G, S, KT);
                }
            }
    printf("%d failures\n", fails);
    return fails != 0;
}
