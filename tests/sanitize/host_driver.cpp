// Sanitizer driver for the library's host helpers (csrc/kq_host.cpp): built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py and run on the CPU.  It calls every host helper
// on exactly sized buffers (one and many factor sets, in-place folding,
// singular and non-finite factors, empty and bad shapes) and checks the
// status codes.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kroquant.h"

#define CHECK(expr, want)                                                                                          \
    do {                                                                                                           \
        int got_ = (expr);                                                                                         \
        if (got_ != (want)) {                                                                                      \
            std::fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #expr, got_, (want)); \
            std::exit(1);                                                                                          \
        }                                                                                                          \
    } while (0)

static uint32_t rng_state = 12345u;
static float urand()
{
    rng_state = rng_state * 1664525u + 1013904223u; // LCG: test inputs only
    return (float)((rng_state >> 8) & 0xFFFF) / 65536.0f - 0.5f;
}

int main()
{
    for (int64_t nT : {1, 2, 36, 384}) {
        std::vector<float> f(nT * 20), inv(nT * 20), K(nT * 1024), Ki(nT * 1024), lu(nT * 15), g(nT * 20);
        for (int64_t i = 0; i < nT * 20; ++i)
            f[i] = ((i % 4 == 0 || i % 4 == 3) ? 1.0f : 0.0f) + 0.3f * urand();
        for (int64_t i = 0; i < nT * 15; ++i)
            lu[i] = (i % 3 == 0) ? 0.7f + 0.2f * urand() : urand();
        CHECK(kq_factor_inverse(f.data(), nT, inv.data()), KQ_OK);
        CHECK(kq_block_matrix(f.data(), nT, K.data()), KQ_OK);
        CHECK(kq_block_inverse(f.data(), nT, Ki.data()), KQ_OK);
        CHECK(kq_lu_factors(lu.data(), nT, g.data()), KQ_OK);
        for (int64_t N : {1, 3, 17}) {
            const int64_t d = 32 * nT;
            std::vector<float> W(N * d), Wo(N * d);
            for (auto &w : W)
                w = urand();
            CHECK(kq_fold_weight(W.data(), N, d, f.data(), nT, Wo.data()), KQ_OK);
            CHECK(kq_fold_weight(W.data(), N, d, f.data(), nT, W.data()), KQ_OK); // in place
            CHECK(kq_fold_weight(W.data(), N, d + 16, f.data(), nT, Wo.data()), KQ_ERR_SHAPE);
            CHECK(kq_fold_weight(W.data(), N, d, f.data(), nT + 1, Wo.data()), KQ_ERR_SHAPE);
        }
    }
    // singular, non-finite and bad arguments
    float sing[20] = {1, 2, 2, 4, 1, 0, 0, 1, 1, 0, 0, 1, 1, 0, 0, 1, 1, 0, 0, 1};
    float out[1024];
    CHECK(kq_factor_inverse(sing, 1, out), KQ_ERR_SINGULAR);
    CHECK(kq_block_inverse(sing, 1, out), KQ_ERR_SINGULAR);
    float nonfin[20] = {NAN, 0, 0, 1, 1, 0, 0, 1, 1, 0, 0, 1, 1, 0, 0, 1, 1, 0, 0, 1};
    CHECK(kq_factor_inverse(nonfin, 1, out), KQ_ERR_SINGULAR);
    float lu0[15] = {0, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1};
    CHECK(kq_lu_factors(lu0, 1, out), KQ_ERR_SINGULAR);
    CHECK(kq_factor_inverse(nullptr, 1, out), KQ_ERR_ARG);
    CHECK(kq_block_matrix(sing, -1, out), KQ_ERR_ARG);
    std::puts("host driver ok");
    return 0;
}
