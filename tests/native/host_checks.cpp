// CPU check of libattnres's host-side validation and planning, built with g++
// under -fsanitize=address,undefined (test code).  It drives every path of the
// validator with fake, never-dereferenced addresses, at every snapshot count
// 0..13 with and without the second addend, and checks the status codes.  A
// stack or heap overrun anywhere in that code aborts the run.
#include "attnres_host.hpp"
#include "attnres.h"

#include <cstdio>
#include <cstdlib>

using namespace attnres;

static int failures = 0;

#define EXPECT(cond)                                                                      \
    do {                                                                                  \
        if (!(cond)) {                                                                    \
            std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);          \
            ++failures;                                                                   \
        }                                                                                 \
    } while (0)

static const void* at(uintptr_t a) { return reinterpret_cast<const void*>(a); }

int main()
{
    const uintptr_t base = uintptr_t(1) << 40;
    const int64_t M = 4, H = 7168;
    const uintptr_t row = uintptr_t(M * H * 2);
    const void* snaps[ATTNRES_MAX_SNAPSHOTS + 1];
    for (int s = 0; s <= ATTNRES_MAX_SNAPSHOTS; ++s)
        snaps[s] = at(base + (uintptr_t)(10 + s) * row);
    const void* prefix = at(base);
    const void* add = at(base + row);
    const void* add2 = at(base + 2 * row);
    const void* query = at(base + 3 * row);
    const void* gamma = at(base + 3 * row + 32768); // query: 14336 bytes at 3*row
    const void* outp = at(base + 4 * row);
    const void* outn = at(base + 5 * row);

    for (int with2 = 0; with2 < 2; ++with2) {
        for (int n = 0; n <= ATTNRES_MAX_SNAPSHOTS + 1; ++n) {
            const void* a2 = with2 ? add2 : nullptr;
            const int want = n <= ATTNRES_MAX_SNAPSHOTS ? ATTNRES_OK : ATTNRES_EUNSUPPORTED;
            EXPECT(validate_fwd(prefix, add, a2, snaps, n, query, gamma, 1e-6f, M, H, outp, outn) == want);
            // in place is allowed
            EXPECT(validate_fwd(prefix, add, a2, snaps, n, query, gamma, 1e-6f, M, H, prefix, outn) == want);
            if (n >= 1 && n <= ATTNRES_MAX_SNAPSHOTS) {
                // out_norm equal to the last snapshot
                EXPECT(validate_fwd(prefix, add, a2, snaps, n, query, gamma, 1e-6f, M, H, outp,
                                    snaps[n - 1]) == ATTNRES_EALIAS);
                // out_prefix inside the last snapshot
                EXPECT(validate_fwd(prefix, add, a2, snaps, n, query, gamma, 1e-6f, M, H,
                                    at(reinterpret_cast<uintptr_t>(snaps[n - 1]) + 4096), outn) ==
                       ATTNRES_EALIAS);
            }
            // the optional mixture output: valid when disjoint, aliasing rejected
            const void* outm = at(base + 6 * row);
            EXPECT(validate_fwd(prefix, add, a2, snaps, n, query, gamma, 1e-6f, M, H, outp, outn, outm) == want);
            if (n <= ATTNRES_MAX_SNAPSHOTS) {
                EXPECT(validate_fwd(prefix, add, a2, snaps, n, query, gamma, 1e-6f, M, H, outp, outn, outp) ==
                       ATTNRES_EALIAS);
                EXPECT(validate_fwd(prefix, add, a2, snaps, n, query, gamma, 1e-6f, M, H, outp, outn,
                                    at(base + 5 * row + 16)) == ATTNRES_EALIAS);
                EXPECT(validate_fwd(prefix, add, a2, snaps, n, query, gamma, 1e-6f, M, H, outp, outn,
                                    at(base + 6 * row + 8)) == ATTNRES_EINVAL);
                if (n >= 1)
                    EXPECT(validate_fwd(prefix, add, a2, snaps, n, query, gamma, 1e-6f, M, H, outp, outn,
                                        snaps[n - 1]) == ATTNRES_EALIAS);
            }
            Plan pl;
            for (int fv = 0; fv <= 3; ++fv)
                for (int fp = 0; fp <= 9; ++fp) {
                    if (!valid_override(fv, fp))
                        continue;
                    for (int64_t m : {int64_t(1), int64_t(8), int64_t(64), int64_t(65), int64_t(512),
                                      int64_t(513), int64_t(1) << 21})
                        for (int64_t h : {int64_t(8), int64_t(520), int64_t(896), int64_t(2048),
                                          int64_t(3584), int64_t(7168), int64_t(8192), int64_t(16384)}) {
                            const int rc = make_plan(m, n, h, fv, fp, pl);
                            if (rc == ATTNRES_OK) {
                                EXPECT(pl.threads % 64 == 0 && pl.threads >= 64 && pl.threads <= 1024);
                                EXPECT(pl.grid >= 1);
                                EXPECT((int64_t)pl.threads * pl.vpt * pl.chunks * 8 >= h);
                                if (n > MAX_SNAP)
                                    EXPECT((pl.variant == 1 && (pl.vpt == 2 || pl.vpt == 4)) ||
                                           (pl.variant == 2 && n <= MAX_SPLIT_SNAP && pl.threads <= 128) ||
                                           (pl.variant == 2 && n > MAX_SPLIT_SNAP && n <= MAX_SPLIT_LONG_SNAP &&
                                            ((pl.threads == 128 && pl.vpt == 1) ||
                                             (pl.threads == 256 && pl.vpt == 2)) &&
                                            pl.chunks <= SPLIT_LONG_MAX_CHUNKS &&
                                            (int64_t)pl.chunks * (pl.threads / 2) * 8 >= h));
                                // the single-group table is built for at most SHORT_WG_THREADS
                                if (pl.single_group)
                                    EXPECT(pl.variant == 1 && pl.vpt == 1 && pl.threads <= SHORT_WG_THREADS &&
                                           m * pl.threads <= SHORT_WG_MAX_THREADS_TOTAL);
                                if (pl.variant == 2)
                                    EXPECT(m <= MAX_SPLIT_TOKENS && pl.chunks <= MAX_CHUNKS &&
                                           pl.grid == 8 * pl.chunks * ((m + 7) / 8) &&
                                           pl.threads <= 512 && pl.split_slots == m &&
                                           pl.split_threads == pl.threads &&
                                           pl.chunks <= (n > MAX_SPLIT_SNAP ? SPLIT_LONG_MAX_CHUNKS
                                                         : pl.threads <= 128 ? MAX_CHUNKS : 8));
                                // the hybrid: W on [0, split_base), one workgroup per token, 1-, 2- or
                                // 4-wave chunks on the rest (one pass of sources), chunks of a token on
                                // one workgroup id mod 8
                                if (pl.variant == 3)
                                    EXPECT(n <= MAX_SNAP && pl.vpt == 2 && pl.threads <= 512 &&
                                           pl.threads >= pl.split_threads &&
                                           (int64_t)pl.threads * 2 * 8 >= h && pl.split_base % 8 == 0 &&
                                           pl.wg_blocks == pl.split_base && pl.split_base <= HYBRID_WG_TOKENS &&
                                           pl.split_base < m && m - pl.split_base <= MAX_SPLIT_TOKENS &&
                                           pl.split_slots == m - pl.split_base &&
                                           (pl.split_threads == 64 || pl.split_threads == 128 ||
                                            pl.split_threads == 256 || pl.split_threads == pl.threads) &&
                                           pl.chunks <= MAX_CHUNKS &&
                                           (int64_t)pl.chunks * pl.split_threads * 8 >= h &&
                                           (int64_t)(pl.chunks - 1) * pl.split_threads * 8 < h &&
                                           pl.grid == pl.split_base + 8 * pl.chunks * ((pl.split_slots + 7) / 8));
                                if (pl.variant == 1)
                                    EXPECT(pl.split_slots == 0);
                            } else {
                                EXPECT(fv != 0 || h > 8192); // automatic always finds a plan
                            }
                        }
                }
        }
    }
    // kernel W's single-group form: short rows, up to 131072 threads per call
    {
        Plan pl;
        EXPECT(make_plan(1024, 12, 896, 0, 0, pl) == ATTNRES_OK && pl.variant == 1 && pl.threads == 128 &&
               pl.single_group);
        EXPECT(make_plan(1025, 12, 896, 0, 0, pl) == ATTNRES_OK && pl.variant == 1 && !pl.single_group);
        EXPECT(make_plan(512, 8, 2048, 0, 0, pl) == ATTNRES_OK && pl.threads == 256 && pl.single_group);
        EXPECT(make_plan(513, 8, 2048, 0, 0, pl) == ATTNRES_OK && pl.variant == 1 && !pl.single_group);
        EXPECT(make_plan(1, 12, 3584, 0, 0, pl) == ATTNRES_OK && pl.variant == 2);
        EXPECT(make_plan(1, 3, 3584, 0, 0, pl) == ATTNRES_OK && pl.variant == 1 && !pl.single_group);
        EXPECT(make_plan(1, 4, 3584, 0, 0, pl) == ATTNRES_OK && pl.variant == 2 && pl.threads == 64);
        EXPECT(make_plan(1, 12, 7168, 1, 1, pl) == ATTNRES_OK && pl.threads == 896 && !pl.single_group);
        EXPECT(make_plan(1, 13, 896, 1, 0, pl) == ATTNRES_OK && pl.vpt == 2 && !pl.single_group);
    }
    // the hybrid just past the CU count, automatic at H = 7168 for one pass of sources
    {
        Plan pl;
        EXPECT(make_plan(256, 12, 7168, 0, 0, pl) == ATTNRES_OK && pl.variant == 1);
        EXPECT(make_plan(257, 12, 7168, 0, 0, pl) == ATTNRES_OK && pl.variant == 3 && pl.split_base == 256 &&
               pl.chunks == 14 && pl.split_threads == 64 && pl.grid == 256 + 112);
        EXPECT(make_plan(272, 12, 7168, 0, 0, pl) == ATTNRES_OK && pl.chunks == 14 && pl.grid == 256 + 224);
        EXPECT(make_plan(273, 12, 7168, 0, 0, pl) == ATTNRES_OK && pl.chunks == 7 && pl.split_threads == 128);
        EXPECT(make_plan(288, 12, 7168, 0, 0, pl) == ATTNRES_OK && pl.chunks == 7 && pl.grid == 256 + 224);
        EXPECT(make_plan(289, 12, 7168, 0, 0, pl) == ATTNRES_OK && pl.chunks == 4 && pl.split_threads == 256);
        EXPECT(make_plan(320, 1, 7168, 0, 0, pl) == ATTNRES_OK && pl.variant == 3 &&
               pl.chunks == 4 && pl.split_threads == 256 && pl.grid == 512);
        EXPECT(make_plan(260, 12, 8192, 0, 0, pl) == ATTNRES_OK && pl.chunks == 16 && pl.threads == 512);
        EXPECT(make_plan(300, 12, 7168, 3, 1, pl) == ATTNRES_OK && pl.chunks == 14 && pl.split_threads == 64);
        EXPECT(make_plan(300, 12, 7168, 3, 8, pl) == ATTNRES_OK && pl.chunks == 2 && pl.split_threads == 448);
        EXPECT(make_plan(321, 12, 7168, 0, 0, pl) == ATTNRES_OK && pl.variant == 3 && pl.chunks == 2 &&
               pl.split_threads == 448 && pl.grid == 256 + 8 * 2 * 9);
        EXPECT(make_plan(352, 4, 8192, 0, 0, pl) == ATTNRES_OK && pl.variant == 3 && pl.chunks == 2 &&
               pl.split_threads == 512);
        EXPECT(make_plan(300, 12, 7168, 3, 7, pl) == ATTNRES_EINVAL);
        EXPECT(make_plan(HYBRID_MAX_TOKENS + 1, 12, 7168, 0, 0, pl) == ATTNRES_OK && pl.variant == 1);
        EXPECT(make_plan(300, 13, 7168, 0, 0, pl) == ATTNRES_OK && pl.variant == 1);
        EXPECT(make_plan(300, 12, 896, 0, 0, pl) == ATTNRES_OK && pl.variant == 1);
        EXPECT(make_plan(20, 5, 7168, 3, 0, pl) == ATTNRES_OK && pl.variant == 3 && pl.split_base == 8);
        EXPECT(make_plan(15, 5, 7168, 3, 0, pl) == ATTNRES_OK && pl.split_base == 0 && pl.wg_blocks == 0);
        EXPECT(make_plan(20, 13, 7168, 3, 0, pl) == ATTNRES_EINVAL);
        EXPECT(make_plan(20, 5, 896, 3, 0, pl) == ATTNRES_EINVAL);
    }
    EXPECT(validate_fwd(nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr, 1e-6f, 0, H, nullptr,
                        nullptr) == ATTNRES_OK);
    EXPECT(validate_add(prefix, add, outp, 1000) == ATTNRES_OK);
    EXPECT(validate_add(prefix, add, prefix, 1000) == ATTNRES_OK);
    EXPECT(validate_add(prefix, add, at(base + 16), 1000) == ATTNRES_EALIAS);
    EXPECT(validate_add(nullptr, nullptr, nullptr, 0) == ATTNRES_OK);
    std::printf("host checks: %d failures\n", failures);
    return failures ? 1 : 0;
}
