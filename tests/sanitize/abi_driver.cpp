// Host-only driver for the sanitizer build of the library (AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code): every call here is a
// query or is refused by argument validation before any HIP call, so it
// runs without a GPU.  Exit status 0 when every check holds.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/mttkrp.h"

static int fails = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++fails;                                                     \
        }                                                                \
    } while (0)

int main()
{
    CHECK(mttkrp_selftest() == 0);
    for (int c = 1; c >= -9; --c) CHECK(mttkrp_strerror(c) != nullptr);

    // planning and workspace queries over a deterministic spread of shapes
    uint64_t s = 12345;
    auto rnd = [&](int lo, int hi) {
        s = s * 6364136223846793005ull + 1442695040888963407ull;
        return lo + (int)((s >> 33) % (uint64_t)(hi - lo + 1));
    };
    int planned = 0;
    for (int t = 0; t < 3000; ++t) {
        const int d = rnd(3, 5);
        int64_t dims[5];
        for (int m = 0; m < d; ++m) dims[m] = rnd(1, t % 7 == 0 ? 600 : 90);
        const int64_t R = t % 11 == 0 ? rnd(1, 2100) : rnd(1, 140);
        const int eb = (t & 1) ? 8 : 4;
        for (int n = 0; n < d; ++n) {
            mttkrp_plan_info info;
            const int st = mttkrp_plan(dims, d, R, n, eb, &info);
            CHECK(st == MTTKRP_OK || st == MTTKRP_ERANGE);
            if (st) continue;
            ++planned;
            CHECK(info.launchable == 1);
            CHECK(info.grid >= 8 && info.grid % 8 == 0);
            CHECK(info.model_s >= info.t_inf_s * (1 - 1e-12));
            size_t ws = 0;
            CHECK(mttkrp_workspace_bytes(dims, d, R, n, eb, &ws) == MTTKRP_OK);
            CHECK(ws == info.ws_bytes);
        }
        size_t all = 0, als = 0;
        const int sa = mttkrp_all_workspace_bytes(dims, d, R, eb, &all);
        CHECK(sa == MTTKRP_OK || sa == MTTKRP_ERANGE);
        const int sl = cp_als_workspace_bytes(dims, d, R, eb, &als);
        CHECK(sl == MTTKRP_OK || sl == MTTKRP_ERANGE);
    }
    CHECK(planned > 5000);

    // validation before any HIP call (pointers are never dereferenced)
    void *const fake = reinterpret_cast<void *>(0x7F0000001000ull);
    void *const mis = reinterpret_cast<void *>(0x7F0000001008ull);
    const int64_t d3[3] = {4, 5, 6};
    const double *f3[3] = {(const double *)fake, (const double *)fake, (const double *)fake};
    CHECK(mttkrp_f64(nullptr, d3, 3, f3, 3, 0, (double *)fake, nullptr, 0, nullptr) == MTTKRP_EINVAL);
    CHECK(mttkrp_f64((const double *)fake, d3, 7, f3, 3, 0, (double *)fake, nullptr, 0, nullptr) ==
          MTTKRP_EORDER);
    CHECK(mttkrp_f64((const double *)mis, d3, 3, f3, 3, 0, (double *)fake, nullptr, 0, nullptr) ==
          MTTKRP_EALIGN);
    CHECK(mttkrp_f64((const double *)fake, d3, 3, f3, 0, 0, (double *)fake, nullptr, 0, nullptr) ==
          MTTKRP_EINVAL);
    const int64_t huge[3] = {INT64_C(1) << 40, INT64_C(1) << 40, 4};
    CHECK(mttkrp_f64((const double *)fake, huge, 3, f3, 3, 0, (double *)fake, nullptr, 0, nullptr) ==
          MTTKRP_ERANGE);
    const int64_t c2[3] = {256, 256, 256};
    CHECK(mttkrp_f64((const double *)fake, c2, 3, f3, 32, 2, (double *)fake, nullptr, 0, nullptr) ==
          MTTKRP_EWORKSPACE);
    double *outs[3] = {(double *)fake, (double *)mis, (double *)fake};
    CHECK(mttkrp_all_f64((const double *)fake, d3, 3, f3, 3, outs, nullptr, 0, nullptr) ==
          MTTKRP_EALIGN);
    double fit[4];
    int done = 0;
    double *fw[3] = {(double *)fake, (double *)fake, (double *)fake};
    CHECK(cp_als_f64((const double *)fake, d3, 3, 5000, fw, (double *)fake, 4, 0.0, fit, &done, fake,
                     1 << 20, nullptr) == MTTKRP_ERANGE);
    CHECK(cp_als_f64((const double *)fake, d3, 3, 3, fw, (double *)fake, 4, 0.0, fit, &done, fake, 16,
                     nullptr) == MTTKRP_EWORKSPACE);
    // the allocation-free entry refuses a plan larger than its scratch array
    const int64_t big[3] = {2048, 512, 512};
    const void *fv[3] = {fake, fake, fake};
    CHECK(mttkrp_noalloc(fake, big, 3, fv, 2000, 0, fake, 8, nullptr) == MTTKRP_ESCRATCH);
    CHECK(mttkrp_noalloc(fake, big, 3, fv, 2000, 0, fake, 3, nullptr) == MTTKRP_EINVAL);
    // the forced-tile override: parsed, applied, refused when malformed
    setenv("MTTKRP_FORCE_TILE", "4,2,8", 1);
    mttkrp_plan_info info;
    CHECK(mttkrp_plan(c2, 3, 32, 0, 8, &info) == MTTKRP_OK && info.mb == 4 && info.nb == 2 &&
          info.waves == 8);
    setenv("MTTKRP_FORCE_TILE", "4,2,8,9", 1);
    CHECK(mttkrp_plan(c2, 3, 32, 0, 8, &info) == MTTKRP_EINVAL);
    unsetenv("MTTKRP_FORCE_TILE");
    // probes: argument checks only
    CHECK(mttkrp_probe_read(nullptr, 16, (uint32_t *)fake, nullptr) == MTTKRP_EINVAL);
    CHECK(mttkrp_probe_mfma(8, 0, (double *)fake, nullptr) == MTTKRP_EINVAL);

    std::printf("abi driver: %d plans, %d failed checks\n", planned, fails);
    return fails ? 1 : 0;
}
