// Host driver for the sanitizer build of the C ABI's host code (AddressSanitizer +
// UndefinedBehaviorSanitizer on the host side only): the pure host helpers over their whole
// argument ranges, and every entry point's argument checks, which return before any launch.
// A host array the library reads (the fan-out of a lookup) is allocated at its exact length, so
// a read past its end is reported.  Any sanitizer report or unexpected return code aborts.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "specverify.h"

static int fails = 0, checks = 0;
#define EXPECT_RC(call, want)                                                              \
    do {                                                                                   \
        const int rc_ = (call);                                                            \
        ++checks;                                                                          \
        if (rc_ != (want)) {                                                               \
            std::printf("line %d: %s returned %d, expected %d\n", __LINE__, #call, rc_, (int)(want)); \
            ++fails;                                                                       \
        }                                                                                  \
    } while (0)

int main() {
    void* fake = reinterpret_cast<void*>(0x1000);  // never dereferenced on these paths
    int32_t* fi = static_cast<int32_t*>(fake);
    const spec_params* fp = static_cast<const spec_params*>(fake);
    // workspace sizes
    for (int B : {-1, 0, 1, 16, 1000})
        for (int K : {0, 1, 5, 63, 64, 100})
            for (int V : {0, 1, 2048, 128256, 262144, 262152}) (void)spec_workspace_bytes(B, K, V);
    // fan-out over its whole domain; the output is exactly K + 1 entries
    for (int K = 1; K <= 65; ++K)
        for (int budget : {0, 1, 32, 1000, 100000}) {
            std::vector<int32_t>* out = new std::vector<int32_t>(K + 1);
            const int rc = saguaro_fanout(K, budget, 0.7, 1.0, out->data());
            ++checks;
            if ((K <= 64) != (rc == SPEC_OK)) {
                std::printf("fanout K=%d budget=%d rc=%d\n", K, budget, rc);
                ++fails;
            }
            if (rc == SPEC_OK) {
                long sum = 0;
                for (int v : *out) sum += v;
                if (sum != budget) {
                    std::printf("fanout K=%d budget=%d sums to %ld\n", K, budget, sum);
                    ++fails;
                }
            }
            delete out;
        }
    for (double a : {0.0, 1.0, -0.5, 0.999999}) {
        std::vector<int32_t> out(6);
        EXPECT_RC(saguaro_fanout(5, 32, a, 1.0, out.data()), (a > 0.0 && a < 1.0) ? SPEC_OK : SPEC_EINVAL);
    }
    EXPECT_RC(saguaro_fanout(5, 32, 0.7, -1.0, fi), SPEC_EINVAL);
    EXPECT_RC(saguaro_fanout(5, 32, 0.7, 1.0, nullptr), SPEC_EINVAL);
    // spec_verify argument checks (all before any launch)
    const size_t ws = spec_workspace_bytes(16, 5, 4096);
    EXPECT_RC(spec_verify(fake, 5, nullptr, SPEC_BF16, 16, 5, 4096, fp, 4, 0.3f, fi, 1, 0, 0, fi, fi, nullptr, nullptr,
                          fake, ws, nullptr), SPEC_EINVAL);
    EXPECT_RC(spec_verify(fake, 5, fake, SPEC_BF16, 0, 5, 4096, fp, 4, 0.3f, fi, 1, 0, 0, fi, fi, nullptr, nullptr,
                          fake, ws, nullptr), SPEC_EINVAL);
    EXPECT_RC(spec_verify(fake, 7, fake, SPEC_BF16, 16, 5, 4096, fp, 4, 0.3f, fi, 1, 0, 0, fi, fi, nullptr, nullptr,
                          fake, ws, nullptr), SPEC_EINVAL);
    EXPECT_RC(spec_verify(fake, 5, fake, SPEC_BF16, 16, 5, 4096, fp, 65, 0.3f, fi, 1, 0, 0, fi, fi, nullptr, nullptr,
                          fake, ws, nullptr), SPEC_EINVAL);
    EXPECT_RC(spec_verify(fake, 5, fake, SPEC_BF16, 16, 5, 4096, fp, 4, 1.5f, fi, 1, 0, 0, fi, fi, nullptr, nullptr,
                          fake, ws, nullptr), SPEC_EINVAL);
    EXPECT_RC(spec_verify(fake, 5, fake, SPEC_BF16, 16, 5, 4096, fp, 4, 0.3f, fi, 1, 0, 64, fi, fi, nullptr, nullptr,
                          fake, ws, nullptr), SPEC_EINVAL);
    EXPECT_RC(spec_verify(fake, 5, fake, 7, 16, 5, 4096, fp, 4, 0.3f, fi, 1, 0, 0, fi, fi, nullptr, nullptr, fake, ws,
                          nullptr), SPEC_EDTYPE);
    EXPECT_RC(spec_verify(fake, 5, fake, SPEC_BF16, 16, 5, 4096, fp, 4, 0.3f, fi, 1, 0, 0, fi, fi, nullptr, nullptr,
                          fake, ws - 1, nullptr), SPEC_EWORKSPACE);
    // pyramid_verify
    EXPECT_RC(pyramid_verify(fake, 5, fake, SPEC_BF16, 16, 5, 4096, fp, 0, 1.0f, nullptr, fi, 1, 0, 0, fi, fi, nullptr,
                             nullptr, nullptr, fake, ws, nullptr), SPEC_EINVAL);
    EXPECT_RC(pyramid_verify(fake, 5, fake, SPEC_BF16, 16, 5, 4096, fp, 0, 1.0f, (const float*)fake, fi, 1, 0, 128, fi,
                             fi, nullptr, nullptr, nullptr, fake, ws, nullptr), SPEC_EINVAL);
    EXPECT_RC(pyramid_verify(fake, 5, fake, SPEC_BF16, 16, 5, 4096, fp, 0, 1.0f, (const float*)fake, fi, 1, 0, 0, fi, fi,
                             nullptr, nullptr, nullptr, fake, 0, nullptr), SPEC_EWORKSPACE);
    // saguaro_verify_cache: bad fan-out arguments, a fan-out past the list limit, a small workspace
    const size_t ws6 = spec_workspace_bytes(16, 5, 4096);
    std::vector<int32_t> fan(6);
    EXPECT_RC(saguaro_verify_cache(fake, fake, SPEC_BF16, 16, 5, 4096, fp, 4, 0.3f, fi, 1, 0, 0, 32, 1.0, 1.0, fan.data(),
                                   fi, fi, nullptr, nullptr, fi, fake, ws6, nullptr), SPEC_EINVAL);
    EXPECT_RC(saguaro_verify_cache(fake, fake, SPEC_BF16, 16, 5, 4096, fp, 4, 0.3f, fi, 1, 0, 0, 100000, 0.7, 1.0,
                                   fan.data(), fi, fi, nullptr, nullptr, fi, fake, ws6, nullptr), SPEC_EINVAL);
    EXPECT_RC(saguaro_verify_cache(fake, fake, SPEC_BF16, 16, 5, 4096, fp, 4, 0.3f, fi, 1, 0, 2, 32, 0.7, 1.0,
                                   fan.data(), fi, fi, nullptr, nullptr, fi, fake, ws6, nullptr), SPEC_EINVAL);
    EXPECT_RC(saguaro_verify_cache(fake, fake, SPEC_BF16, 16, 5, 4096, fp, 4, 0.3f, fi, 1, 0, 0, 32, 0.7, 1.0,
                                   fan.data(), fi, fi, nullptr, nullptr, fi, fake, ws6 - 256, nullptr), SPEC_EWORKSPACE);
    // saguaro_cache_build: budget 0 returns after writing the K + 1 fan-out entries to the host
    EXPECT_RC(saguaro_cache_build(fake, SPEC_BF16, 16, 5, 4096, fi, 0, 0.7, 1.0, fan.data(), fi, nullptr), SPEC_OK);
    EXPECT_RC(saguaro_cache_build(fake, SPEC_BF16, 16, 5, 4096, fi, 32, 0.0, 1.0, fan.data(), fi, nullptr), SPEC_EINVAL);
    EXPECT_RC(saguaro_cache_build(fake, 3, 16, 5, 4096, fi, 32, 0.7, 1.0, fan.data(), fi, nullptr), SPEC_EDTYPE);
    // saguaro_cache_lookup: the fan-out is read at exactly K + 1 entries (the last one invalid)
    for (int K : {1, 5, 64}) {
        std::vector<int32_t>* f = new std::vector<int32_t>(K + 1, 2);
        f->back() = -1;
        EXPECT_RC(saguaro_cache_lookup(0, fi, f->data(), K, 4, fi, fi, fi, (uint8_t*)fake, fi, nullptr), SPEC_EINVAL);
        delete f;
    }
    {
        std::vector<int32_t>* shape = new std::vector<int32_t>{0, 7};
        EXPECT_RC(saguaro_cache_lookup(1, fi, shape->data(), 0, 4, fi, fi, fi, (uint8_t*)fake, fi, nullptr), SPEC_EINVAL);
        delete shape;
        std::vector<int32_t>* f = new std::vector<int32_t>(6, 1);
        EXPECT_RC(saguaro_cache_lookup(0, fi, f->data(), 65, 4, fi, fi, fi, (uint8_t*)fake, fi, nullptr), SPEC_EINVAL);
        EXPECT_RC(saguaro_cache_lookup(2, fi, f->data(), 5, 4, fi, fi, fi, (uint8_t*)fake, fi, nullptr), SPEC_EINVAL);
        delete f;
    }
    // the other entry points' checks
    EXPECT_RC(saguaro_backup_plan(0, (const uint8_t*)fake, fi, 2, fi, fi, nullptr), SPEC_EINVAL);
    EXPECT_RC(saguaro_downweight(fake, 4, SPEC_BF16, 16, 5, 4096, fp, 4, 0.3f, fi, nullptr, nullptr, nullptr, nullptr),
              SPEC_EINVAL);
    EXPECT_RC(saguaro_downweight(fake, 5, 9, 16, 5, 4096, fp, 4, 0.3f, fi, nullptr, nullptr, nullptr, nullptr),
              SPEC_EDTYPE);
    for (int kappa : {0, 1, 8, 16, 17})
        for (int V : {0, 1, 151936, 1 << 19, (1 << 19) + 1}) (void)mirror_signpost_workspace_bytes(64, V, kappa);
    EXPECT_RC(mirror_signposts(fake, SPEC_BF16, 64, 151936, 17, fi, (float*)fake, nullptr, nullptr, fake, 1 << 20,
                               nullptr), SPEC_EINVAL);
    EXPECT_RC(mirror_signposts(fake, SPEC_BF16, 64, 151936, 8, fi, (float*)fake, nullptr, nullptr, fake, 0, nullptr),
              SPEC_EWORKSPACE);
    EXPECT_RC(mirror_tree_lookup(fi, fi, 4, 16, 0, fi, fi, fi, fi, (uint8_t*)fake, fi, nullptr), SPEC_EINVAL);
    std::printf("capi driver: %d checks, %d failures\n", checks, fails);
    return fails ? 1 : 0;
}
