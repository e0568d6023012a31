// Host-side argument validation and dispatch planning (see attnres_host.hpp).
#include "attnres_host.hpp"

#include "attnres.h"

#include <algorithm>
#include <cmath>

namespace attnres {

static_assert(MAX_SNAP_LONG == ATTNRES_MAX_SNAPSHOTS, "snapshot limit mismatch");
static_assert(MAX_HIDDEN == ATTNRES_MAX_HIDDEN, "hidden limit mismatch");

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na && nb && x < y + nb && y < x + na;
}

int round_up64(int64_t x) { return (int)((x + 63) / 64 * 64); }

bool plan_wg(int64_t M, int nvec, int vpt, Plan& pl)
{
    if (vpt == 0)
        vpt = nvec <= 512 ? 1 : nvec <= 1024 ? 2 : 4;
    if (vpt != 1 && vpt != 2 && vpt != 4)
        return false;
    const int maxb = vpt == 1 ? 1024 : 512;
    const int threads = std::max(64, round_up64((nvec + vpt - 1) / vpt));
    if (threads > maxb)
        return false;
    pl = Plan{};
    pl.variant = 1;
    pl.vpt = vpt;
    pl.threads = threads;
    pl.chunks = 1;
    pl.grid = std::min<int64_t>(M, int64_t(1) << 20);
    pl.single_group = vpt == 1 && threads <= SHORT_WG_THREADS && M * threads <= SHORT_WG_MAX_THREADS_TOTAL;
    return true;
}

// Split hidden: `waves` (1, 2 or 4..8) waves per workgroup, one vector per thread, C chunks
// per token; grid = 8 * C * ceil(M / 8) (chunks of a token share an XCD).
bool plan_split(int64_t M, int nvec, int waves, Plan& pl)
{
    if (waves == 0)
        waves = 2;
    if (waves < 1 || waves > 8)
        return false;
    if (waves == 3)
        return false; // 1-2 waves: up to 32 chunks; 4-8 waves: up to 8 chunks
    const int threads = 64 * waves;
    const int chunks = (nvec + threads - 1) / threads;
    if (chunks > (waves <= 2 ? MAX_CHUNKS : 8) || M > MAX_SPLIT_TOKENS)
        return false;
    pl = Plan{};
    pl.variant = 2;
    pl.vpt = 1;
    pl.threads = threads;
    pl.chunks = chunks;
    pl.grid = 8 * (int64_t)chunks * ((M + 7) / 8);
    pl.split_threads = threads;
    pl.split_slots = M;
    return true;
}

// Hybrid: kernel W (two vectors per thread) on the first nw tokens, one
// workgroup each, then split chunks of `waves` waves on the other M - nw
// (waves = 0: the narrowest of 1, 2 and 4 whose chunk workgroups, 8 C per
// group of 8 token slots, number at most HYBRID_WG_TOKENS, else 4): the extra
// tokens spread over as many CUs as there are, in pieces as small as that
// allows, so no CU's W token waits behind much of a chunk (M = 264, N = 12:
// 1-wave 13.60 against 4-wave 15.64 us; M = 288: 2-wave 14.55 against 16.05;
// M = 300 and 320: 4-wave 15.98 and 17.21 against 18.0 and 19.0 for 2-wave).
// nw is a multiple of 8 so the chunks of a token keep one workgroup id mod 8.
// The split kernel's forms for 32..MAX_SPLIT_LONG_SNAP snapshots, at most
// SPLIT_LONG_MAX_CHUNKS chunks per token: waves = 2, chunks of 64 vectors
// with two waves each (each holding half of the sources); waves = 4, chunks
// of 128 vectors (two per lane) with four waves each (a quarter each).
bool plan_split_long(int64_t M, int nvec, int waves, Plan& pl)
{
    if (waves != 2 && waves != 4)
        return false;
    const int width = waves == 2 ? 64 : 128;
    const int chunks = (nvec + width - 1) / width;
    if (chunks > SPLIT_LONG_MAX_CHUNKS || M > MAX_SPLIT_TOKENS)
        return false;
    pl = Plan{};
    pl.variant = 2;
    pl.vpt = waves == 2 ? 1 : 2;
    pl.threads = 64 * waves;
    pl.chunks = chunks;
    pl.grid = 8 * (int64_t)chunks * ((M + 7) / 8);
    pl.split_threads = pl.threads;
    pl.split_slots = M;
    return true;
}

// The form of 32..MAX_SPLIT_LONG_SNAP snapshots the automatic dispatch takes
// for M tokens, or 0 for kernel W's batches.
int split_long_waves(int64_t M, int n, int nvec)
{
    if (nvec < LONG_ROW_VECTORS)
        return M <= SPLIT_LONG_TOKENS ? 2 : 0;
    if (M > (n >= SPLIT_LONG_WIDE_SNAP ? SPLIT_LONG_TOKENS : SPLIT_LONG_TOKENS_LONG_ROWS))
        return 0;
    return nvec <= VERY_LONG_ROW_VECTORS && M <= SPLIT_LONG_PAIR_TOKENS ? 2 : 4;
}

bool plan_hybrid(int64_t M, int nvec, int waves, Plan& pl)
{
    if (nvec <= 512 || nvec > 1024 || M < 1 ||
        !(waves == 0 || waves == 1 || waves == 2 || waves == 4 || waves == HYBRID_HALF_ROW))
        return false;
    const int64_t nw = M > HYBRID_WG_TOKENS ? HYBRID_WG_TOKENS : (M / 2) / 8 * 8;
    const int64_t rest = M - nw;
    if (rest > MAX_SPLIT_TOKENS)
        return false;
    const int64_t groups = (rest + 7) / 8;
    const int threads = round_up64((nvec + 1) / 2);
    if (waves == 0) {
        waves = HYBRID_HALF_ROW;
        for (int w = 1; w <= 4; w *= 2)
            if (8 * (int64_t)((nvec + 64 * w - 1) / (64 * w)) * groups <= HYBRID_WG_TOKENS) {
                waves = w;
                break;
            }
    }
    const int chunk_threads = waves == HYBRID_HALF_ROW ? threads : 64 * waves;
    const int chunks = (nvec + chunk_threads - 1) / chunk_threads;
    pl = Plan{};
    pl.variant = 3;
    pl.vpt = 2;
    pl.threads = threads;
    pl.chunks = chunks;
    pl.split_base = nw;
    pl.split_threads = chunk_threads;
    pl.wg_blocks = (int)nw;
    pl.grid = nw + 8 * (int64_t)chunks * groups;
    pl.split_slots = rest;
    return chunk_threads <= threads && chunks <= MAX_CHUNKS;
}

} // namespace

int validate_sizes(int64_t M, int n, int64_t H)
{
    if (n < 0)
        return ATTNRES_EINVAL;
    if (n > MAX_SNAP_LONG)
        return ATTNRES_EUNSUPPORTED;
    if (M < 0 || M > INT32_MAX || H < 8 || H % 8 != 0 || H > MAX_HIDDEN)
        return ATTNRES_EINVAL;
    return ATTNRES_OK;
}

int validate_fwd(const void* prefix, const void* add, const void* add2, const void* const* snapshots,
                 int n, const void* query, const void* gamma, float eps, int64_t M, int64_t H,
                 const void* out_prefix, const void* out_norm, const void* out_mix)
{
    int rc = validate_sizes(M, n, H);
    if (rc != ATTNRES_OK)
        return rc;
    if (!(eps >= 0.0f) || std::isinf(eps))
        return ATTNRES_EINVAL;
    if (M == 0)
        return ATTNRES_OK; // empty batch: the [M,H] buffers may be empty (NULL)
    if (!prefix || !add || !query || !gamma || !out_prefix || !out_norm)
        return ATTNRES_EINVAL;
    if (n > 0 && !snapshots)
        return ATTNRES_EINVAL;
    for (int s = 0; s < n; ++s)
        if (!snapshots[s] || !aligned16(snapshots[s]))
            return ATTNRES_EINVAL;
    if (!aligned16(prefix) || !aligned16(add) || (add2 && !aligned16(add2)) || !aligned16(query) ||
        !aligned16(gamma) || !aligned16(out_prefix) || !aligned16(out_norm) ||
        (out_mix && !aligned16(out_mix)))
        return ATTNRES_EINVAL;

    // Every read-only buffer other than prefix: add, add2, query, gamma, snapshots.
    const size_t row_bytes = (size_t)M * (size_t)H * 2u, vec_bytes = (size_t)H * 2u;
    const void* ins[4 + MAX_SNAP_LONG];
    size_t sizes[4 + MAX_SNAP_LONG];
    int ni = 0;
    ins[ni] = add, sizes[ni++] = row_bytes;
    if (add2)
        ins[ni] = add2, sizes[ni++] = row_bytes;
    ins[ni] = query, sizes[ni++] = vec_bytes;
    ins[ni] = gamma, sizes[ni++] = vec_bytes;
    for (int s = 0; s < n; ++s)
        ins[ni] = snapshots[s], sizes[ni++] = row_bytes;
    // out_prefix: equal to prefix (in place) or disjoint from it; disjoint from all else
    if (out_prefix != prefix && overlaps(out_prefix, row_bytes, prefix, row_bytes))
        return ATTNRES_EALIAS;
    if (overlaps(out_prefix, row_bytes, out_norm, row_bytes))
        return ATTNRES_EALIAS;
    if (overlaps(out_norm, row_bytes, prefix, row_bytes))
        return ATTNRES_EALIAS;
    for (int i = 0; i < ni; ++i)
        if (overlaps(out_prefix, row_bytes, ins[i], sizes[i]) ||
            overlaps(out_norm, row_bytes, ins[i], sizes[i]))
            return ATTNRES_EALIAS;
    // out_mix (optional): disjoint from every other buffer
    if (out_mix) {
        if (overlaps(out_mix, row_bytes, prefix, row_bytes) ||
            overlaps(out_mix, row_bytes, out_prefix, row_bytes) ||
            overlaps(out_mix, row_bytes, out_norm, row_bytes))
            return ATTNRES_EALIAS;
        for (int i = 0; i < ni; ++i)
            if (overlaps(out_mix, row_bytes, ins[i], sizes[i]))
                return ATTNRES_EALIAS;
    }
    return ATTNRES_OK;
}

bool valid_override(int variant, int param)
{
    switch (variant) {
    case 0: return param == 0;
    case 1: return param == 0 || param == 1 || param == 2 || param == 4;
    case 2: return param >= 0 && param <= 8 && param != 3;
    case 3: return param == 0 || param == 1 || param == 2 || param == 4 || param == HYBRID_HALF_ROW;
    default: return false;
    }
}

int make_plan(int64_t M, int n, int64_t H, int force_variant, int force_param, Plan& pl)
{
    const int nvec = (int)(H / 8);
    // More sources than one pass of kernel W holds: W takes them in batches of
    // MAX_SNAP (instantiated for 2 and 4 vectors per thread); the split kernel
    // takes up to MAX_SPLIT_SNAP in its 1-2-wave family, and up to
    // MAX_SPLIT_LONG_SNAP in its two-wave form (chunks of 64 vectors).
    const bool many = n > MAX_SNAP;
    const int wg_vpt = many ? nvec <= 1024 ? 2 : 4 : 0;
    const bool split_ok = !many || n <= MAX_SPLIT_SNAP;
    const bool split_long = n > MAX_SPLIT_SNAP && n <= MAX_SPLIT_LONG_SNAP;
    if (force_variant == 1) {
        if (many && force_param == 1)
            return ATTNRES_EINVAL;
        return plan_wg(M, nvec, force_param ? force_param : wg_vpt, pl) ? ATTNRES_OK : ATTNRES_EINVAL;
    }
    if (force_variant == 2) {
        if (split_long && (force_param <= 1 || force_param == 4)) {
            int w = force_param == 4 ? 4 : force_param == 1 ? 2 : split_long_waves(M, n, nvec);
            if (w == 0)
                w = nvec <= VERY_LONG_ROW_VECTORS ? 2 : 4;
            return plan_split_long(M, nvec, w, pl) ? ATTNRES_OK : ATTNRES_EINVAL;
        }
        if (!split_ok || (many && force_param > 2))
            return ATTNRES_EINVAL;
        return plan_split(M, nvec, many && force_param == 0 ? 2 : force_param, pl) ? ATTNRES_OK
                                                                                    : ATTNRES_EINVAL;
    }
    if (force_variant == 3)
        return !many && plan_hybrid(M, nvec, force_param, pl) ? ATTNRES_OK : ATTNRES_EINVAL;
    // Automatic, from per-call times of every variant on MI355X (graph
    // replay, inputs cold in HBM, M = 1..512, N = 1..12).  At H = 7168, one
    // pass of sources:
    //  * N >= 6 (two exchanges): 1-wave chunks (14 per token, every chunk's
    //    records in flight at once) up to 48 tokens, and up to 64 with at
    //    most 8 snapshots (M = 64, N = 8: 7.10 against 7.16 us for 4-wave
    //    chunks); otherwise 4-wave chunks up to 64 (N = 10: 7.33 against
    //    7.53 for 1-wave); 1-wave again up to 88 (M = 80, N = 9..11:
    //    7.98-8.57 against 8.21-8.74 for 2-wave; M = 88, N = 8 and 12: 7.85
    //    and 9.10 against 8.03 and 9.25); then up to 96, 2-wave chunks from 8
    //    snapshots on (N = 12, M = 96: 9.46 against 10.02 for W), 1-wave at
    //    N = 7 (7.64 against 7.92 for W), W at N = 6 (7.30 against 7.40);
    //    M = 1, N = 12: 5.07 us; N = 6: 4.62 against 5.40 for the Gram form
    //    in 2-wave chunks;
    //  * 2 <= N <= 5 (the Gram form's one exchange): 1-wave chunks up to 40
    //    tokens at N = 2, 56 at N = 3, 64 from N = 4 on (M = 24, N = 2: 5.00
    //    against 5.13 for 2-wave chunks; M = 48, N = 4: 5.85 against 6.16
    //    for 4-wave chunks; M = 64, N = 2 and 3: W 5.45 and 5.84 against
    //    5.66 and 5.87);
    //  * N = 1: 1-wave chunks up to 8 tokens (M = 1: 4.01 against 4.35 us
    //    for one workgroup per token without add2, 4.11 against 4.62 with it;
    //    M = 8: 4.45 against 4.42 and 4.55 against 4.68; M = 16: 4.53 against
    //    4.46 and 4.63 against 4.73), then one workgroup per token;
    //  * N = 0 at every M: one workgroup per token (M = 1: 3.83 against 3.96
    //    without add2, 4.24 against 4.06 with it; the dispatch may not depend
    //    on add2);
    //  * otherwise one workgroup per token (or the hybrid, below).
    // Rows longer than 8192 (1,536 and 2,048 vectors measured), N <= 12: kernel
    // W's token is one CU's stream of a long row, so the split wins at every
    // N up to 96 tokens, in chunks that keep 6-16 per token: 2-wave up to 16
    // tokens and from 33 to 48, 4-wave from 17 to 32 and from 49 to 96 (H =
    // 16384: M = 1, N = 0: 4.62 against 6.26 us for W; M = 16, N = 1: 5.13
    // against 7.39; M = 32, N = 12: 4-wave 8.22 against 8.68 for 1-wave and
    // 17.40 for W; M = 48, N = 12: 2-wave 10.10 against 10.47 for 4-wave; M =
    // 96, N = 4: 4-wave 9.79 against 11.51 for W; H = 12288, M = 64, N = 8:
    // 2-wave 8.61 against 4-wave 9.02 and W 12.25).
    // More than one pass of sources (up to 31 snapshots, which the 1-2-wave
    // family holds): 1-wave chunks up to 16 tokens and from 33 to 64, 2-wave
    // chunks from 17 to 32 and from 65 to 96, else W's batches (N = 13, 20,
    // 31: M = 1 5.15 against 5.86 us for 2-wave, N = 13; M = 24, N = 31:
    // 2-wave 8.65 against 9.10; M = 64: 1-wave 8.13 / 9.98 / 12.00 against
    // 8.64 / 10.69 / 13.10; M = 96: 2-wave 9.60 / 12.03 / 15.08 against W
    // 10.92 / 14.45 / 19.75; M = 192: W 12.35 / 16.31 / 22.73 against
    // 14.64 / 18.94 / 27.30).  Shorter rows (2 or 7 chunks per token at H =
    // 896 / 3584): 1-wave chunks at every M up to 96 (H = 3584, M = 80, N =
    // 20: 8.13 against 9.72 us for 2-wave and 10.79 for W; H = 896, M = 32,
    // N = 31: 6.72 against 7.24 and 12.25).  Rows longer than 8192: 2-wave
    // chunks except from 17 to 32 tokens, where 1-wave (H = 16384, M = 48,
    // N = 31: 16.76 against 18.34 us for 1-wave; M = 16, N = 20: 8.74
    // against 9.66; H = 12288, M = 32, N = 31: 1-wave 11.65 against 13.00;
    // one token within 0.4 us either way).
    // 32..63 snapshots (split_long_waves): rows of 7168 and more take the
    // split's two-wave form up to 16 tokens (rows of at most 8192) and its
    // four-wave form beyond, up to 64 tokens and up to 96 from 40 snapshots
    // on, else W's batches; shorter rows the two-wave form up to 96 (H =
    // 7168, M = 1, N = 32 / 63: 8.72 / 9.06 against 19.49 / 34.90 us for W
    // and 9.26 / 9.43 in four waves; M = 24, N = 32: four-wave 10.80 against
    // 13.53 two-wave and 19.49 W; M = 96, N = 40: 23.57 against W's 24.36,
    // N = 32: W 20.39 against 22.69; H = 16384, M = 1, N = 63: 9.67 against
    // W's 61.28; M = 64, N = 32: 28.85 against 35.75; M = 96, N = 32: W
    // 37.67 against 40.94; H = 896: two-wave 7.9..9.4 against four-wave
    // 8.6..9.8 up to 96 tokens).
    // Shorter rows (H = 896 ... 4096, N <= 12): a token's rows fit in flight
    // on one CU, and the exchange of a split costs more than it spreads.
    //  * H <= 2048: one workgroup per token everywhere (H = 896, N = 12: 3.88
    //    against 4.90 us for one token, 4.66 against 6.00 for 256);
    //  * H = 3584 / 4096: 1-wave split chunks up to 32 tokens at N = 4, 48
    //    at N = 5..7, 64 at N = 8..11 and 96 at N = 12 (H = 3584, M = 1, N =
    //    6: 4.46 against W 5.26; N = 4: 4.30 against 4.64; M = 48, N = 5:
    //    5.49 against 5.71; N = 6: 5.59 against 5.80; N = 8: 5.73 against
    //    5.92 for 2-wave chunks; M = 96, N = 12: 6.92 against W 7.67);
    //    otherwise W (M = 48, N = 4: 5.17 against 5.34; M = 64, N = 6: 5.71
    //    against 5.77; M = 1, N = 2 and 3: 3.88 and 4.01 against 4.04 and
    //    4.09).
    const bool long_rows = nvec >= LONG_ROW_VECTORS;
    if (split_long) {
        const int w = split_long_waves(M, n, nvec);
        if (w && plan_split_long(M, nvec, w, pl))
            return ATTNRES_OK;
    } else if (many) {
        const bool mid_m = M > SPLIT_SMALL_TOKENS && M <= SPLIT_SMALL_TOKENS_WIDE; // 17..32
        const int waves = !long_rows                      ? 1
                          : nvec > VERY_LONG_ROW_VECTORS ? (mid_m ? 1 : 2)
                          : (M <= SPLIT_SMALL_TOKENS || (M > SPLIT_SMALL_TOKENS_WIDE && M <= SPLIT_MID_TOKENS)) ? 1
                                                                                                              : 2;
        if (M <= SPLIT_WIDE_TOKENS && split_ok && plan_split(M, nvec, waves, pl))
            return ATTNRES_OK;
    } else if (!long_rows) {
        if (nvec > SHORT_ROW_VECTORS && n >= MID_SPLIT_MIN_SNAP && M <= mid_one_wave_tokens(n) &&
            plan_split(M, nvec, 1, pl))
            return ATTNRES_OK;
    } else if (nvec > VERY_LONG_ROW_VECTORS) {
        const int waves = M <= SPLIT_SMALL_TOKENS || (M > SPLIT_SMALL_TOKENS_WIDE && M <= SPLIT_ONE_WAVE_TOKENS) ? 2 : 4;
        if (M <= SPLIT_WIDE_TOKENS && plan_split(M, nvec, waves, pl))
            return ATTNRES_OK;
    } else if (n >= GRAM_MAX_SOURCES) {
        const bool one_wave = M <= SPLIT_ONE_WAVE_TOKENS || (M <= SPLIT_MID_TOKENS && n <= SPLIT_MID_ONE_WAVE_SNAP) ||
                              (M > SPLIT_MID_TOKENS && M <= SPLIT_LATE_ONE_WAVE_TOKENS) ||
                              (n == 7 && M > SPLIT_MID_TOKENS && M <= SPLIT_WIDE_TOKENS);
        if (one_wave && plan_split(M, nvec, 1, pl))
            return ATTNRES_OK;
        if (M <= SPLIT_MID_TOKENS && plan_split(M, nvec, 4, pl))
            return ATTNRES_OK;
        if (n >= 8 && M <= SPLIT_WIDE_TOKENS && plan_split(M, nvec, 2, pl))
            return ATTNRES_OK;
    } else if (n >= 1) {
        if (M <= gram_one_wave_tokens(n) && plan_split(M, nvec, 1, pl))
            return ATTNRES_OK;
    }
    // Just past the CU count, kernel W would give some CUs two whole tokens
    // and the others one; the hybrid gives every CU one W token and a few
    // split chunks of the rest.
    if (long_rows && !many && M > HYBRID_WG_TOKENS && M <= HYBRID_MAX_TOKENS && plan_hybrid(M, nvec, 0, pl))
        return ATTNRES_OK;
    // Prefill-sized calls with long rows: four vectors per thread (256
    // threads; M = 2048, N = 12: 85.98 against 90.48 us for two; M = 4096:
    // 170.3 against 172.2; M = 8192: 343.0 against 345.6; below 2048 tokens
    // two vectors win or tie: M = 512: 23.19 against 23.67).
    const int vpt = !many && long_rows && nvec <= 1024 && M >= PREFILL_WG4_TOKENS ? 4 : wg_vpt;
    if (plan_wg(M, nvec, vpt, pl))
        return ATTNRES_OK;
    return split_ok && plan_split(M, nvec, many ? 2 : 0, pl) ? ATTNRES_OK : ATTNRES_EINVAL;
}

int validate_add(const void* a, const void* b, const void* out, int64_t n)
{
    if (n < 0)
        return ATTNRES_EINVAL;
    if (n == 0)
        return ATTNRES_OK; // nothing to add: the pointers are not examined
    if (!a || !b || !out)
        return ATTNRES_EINVAL;
    if (!aligned16(a) || !aligned16(b) || !aligned16(out))
        return ATTNRES_EINVAL;
    const size_t bytes = (size_t)n * 2u;
    if ((out != a && overlaps(out, bytes, a, bytes)) || (out != b && overlaps(out, bytes, b, bytes)))
        return ATTNRES_EALIAS;
    return ATTNRES_OK;
}

} // namespace attnres
