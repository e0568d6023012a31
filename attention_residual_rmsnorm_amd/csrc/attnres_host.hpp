// Host-side argument validation and dispatch planning of libattnres.
// Plain C++ (no HIP calls, no device code), so it also builds with g++ under
// address/undefined-behaviour sanitizers for CPU tests.
#pragma once

#include <cstddef>
#include <cstdint>

namespace attnres {

constexpr int MAX_SNAP = 12;             // snapshots of one pass (kernel S, and W's batch size)
constexpr int MAX_SNAP_LONG = 64;        // == ATTNRES_MAX_SNAPSHOTS: W in batches of MAX_SNAP
constexpr int MAX_SPLIT_SNAP = 31;       // split hidden, 1-2 waves per workgroup: up to 32 sources
constexpr int MAX_HIDDEN = 16384;        // == ATTNRES_MAX_HIDDEN
constexpr int MAX_SPLIT_TOKENS = 512;    // token slots of the split-hidden scratch
constexpr int MAX_CHUNKS = 32;           // workgroups per token in the split-hidden kernel
// The split kernel's two- and four-wave forms (32..MAX_SPLIT_LONG_SNAP
// snapshots): chunks of 64 vectors with two waves each (wave w holding
// sources 32w .. 32w + 31) or of 128 vectors with four (16 sources each), at
// most SPLIT_LONG_MAX_CHUNKS chunks per token, so that each chunk's 2 (N + 1)
// first-exchange values fit in two pages of 64 records (its own chunk index
// and that index + SPLIT_LONG_MAX_CHUNKS).  Automatic (split_long_waves):
// rows shorter than LONG_ROW_VECTORS the two-wave form up to
// SPLIT_LONG_TOKENS tokens; longer rows the two-wave form up to
// SPLIT_LONG_PAIR_TOKENS tokens (rows of at most VERY_LONG_ROW_VECTORS) and
// the four-wave form beyond, up to SPLIT_LONG_TOKENS_LONG_ROWS tokens, or up
// to SPLIT_LONG_TOKENS from SPLIT_LONG_WIDE_SNAP snapshots on.
constexpr int MAX_SPLIT_LONG_SNAP = 63;
constexpr int SPLIT_LONG_MAX_CHUNKS = MAX_CHUNKS / 2;
constexpr int SPLIT_LONG_TOKENS = 96;
constexpr int SPLIT_LONG_TOKENS_LONG_ROWS = 64;
constexpr int SPLIT_LONG_WIDE_SNAP = 40;
constexpr int SPLIT_LONG_PAIR_TOKENS = 16;
// automatic dispatch (see make_plan) at H >= 7168, one pass of sources:
// N >= GRAM_MAX_SOURCES (two exchanges): 1-wave split chunks up to
// SPLIT_ONE_WAVE_TOKENS tokens, and up to SPLIT_MID_TOKENS with at most
// SPLIT_MID_ONE_WAVE_SNAP snapshots, else 4-wave chunks up to SPLIT_MID_TOKENS;
// 1-wave chunks again up to SPLIT_LATE_ONE_WAVE_TOKENS, then (from
// SPLIT_LATE_ONE_WAVE_TOKENS + 1) 2-wave chunks up to SPLIT_WIDE_TOKENS from 8
// snapshots on and 1-wave chunks at N = 7; 2 <= N < GRAM_MAX_SOURCES (the
// Gram form's one exchange; N = 1 too): 1-wave chunks up to
// gram_one_wave_tokens(N).
// More than one pass of sources (up to MAX_SPLIT_SNAP snapshots): 1-wave
// chunks up to SPLIT_SMALL_TOKENS tokens and from SPLIT_SMALL_TOKENS_WIDE + 1
// to SPLIT_MID_TOKENS, 2-wave chunks otherwise up to SPLIT_WIDE_TOKENS (rows
// shorter than LONG_ROW_VECTORS: 1-wave chunks up to SPLIT_WIDE_TOKENS; rows
// of more than VERY_LONG_ROW_VECTORS: 1-wave chunks from SPLIT_SMALL_TOKENS +
// 1 to SPLIT_SMALL_TOKENS_WIDE, else 2-wave).
constexpr int SPLIT_SMALL_TOKENS = 16;
constexpr int SPLIT_SMALL_TOKENS_WIDE = 32;
constexpr int SPLIT_ONE_WAVE_TOKENS = 48;
constexpr int SPLIT_MID_TOKENS = 64;
constexpr int SPLIT_MID_ONE_WAVE_SNAP = 8;
constexpr int SPLIT_LATE_ONE_WAVE_TOKENS = 88;
constexpr int SPLIT_WIDE_TOKENS = 96;
constexpr int gram_one_wave_tokens(int n) { return n <= 1 ? 8 : n == 2 ? 40 : n == 3 ? 56 : SPLIT_MID_TOKENS; }
// The split kernel's Gram form (one exchange instead of two) serves up to
// GRAM_MAX_SOURCES sources (N <= GRAM_MAX_SOURCES - 1): its 6 + 21 values
// per chunk at N = 5 still fit one polling round with two lanes per value,
// and from 7 sources on the second exchange costs less than the Gram form's
// extra values and arithmetic.
constexpr int GRAM_MAX_SOURCES = 6;
// Rows of at most SHORT_ROW_VECTORS 16-byte vectors (H <= 2048) stay one
// workgroup per token at every M and N <= 12; rows shorter than
// LONG_ROW_VECTORS (H < 7168) are split in 1-wave chunks from N =
// MID_SPLIT_MIN_SNAP on, up to mid_one_wave_tokens(N) tokens; rows of
// LONG_ROW_VECTORS and more follow the rules above.
constexpr int SHORT_ROW_VECTORS = 256;
constexpr int LONG_ROW_VECTORS = 896;
// Rows of more than VERY_LONG_ROW_VECTORS vectors (H > 8192), N <= 12: the
// split in 2-wave chunks up to SPLIT_SMALL_TOKENS tokens and from
// SPLIT_SMALL_TOKENS_WIDE + 1 to SPLIT_ONE_WAVE_TOKENS, 4-wave chunks from
// SPLIT_SMALL_TOKENS + 1 to SPLIT_SMALL_TOKENS_WIDE and from
// SPLIT_ONE_WAVE_TOKENS + 1 to SPLIT_WIDE_TOKENS, at every N.
constexpr int VERY_LONG_ROW_VECTORS = 1024;
constexpr int MID_SPLIT_MIN_SNAP = 4;
constexpr int mid_one_wave_tokens(int n)
{
    return n >= MAX_SNAP ? SPLIT_WIDE_TOKENS : n >= 8 ? SPLIT_MID_TOKENS : n >= 5 ? SPLIT_ONE_WAVE_TOKENS
                                                                            : SPLIT_SMALL_TOKENS_WIDE;
}
// Kernel W's single-group form (one vector per thread, at most
// SHORT_WG_THREADS threads) while M * threads <= SHORT_WG_MAX_THREADS_TOTAL:
// beyond that the form with groups of two keeps more waves per CU and streams
// faster at N = 12 (H = 896, M = 2,048: 13.1 against 14.0 us; up to the bound
// the single group wins, e.g. M = 1,024: 8.8 against 8.9, and H = 2048, M =
// 384: 8.2 against 8.7).
constexpr int SHORT_WG_THREADS = 256;
// Prefill-sized calls (M >= PREFILL_WG4_TOKENS, rows of 513..1024 vectors,
// one pass of sources) take kernel W with four vectors per thread.
constexpr int64_t PREFILL_WG4_TOKENS = 2048;
constexpr int64_t SHORT_WG_MAX_THREADS_TOTAL = 131072;

// The hybrid launch (kernel W's workgroups for the first HYBRID_WG_TOKENS
// tokens, one token each, and split chunks for the rest: the narrowest of 1,
// 2 and 4 waves whose workgroups still number at most HYBRID_WG_TOKENS, one
// per CU next to its W token, else half rows, W's workgroup width), automatic
// for rows of LONG_ROW_VECTORS..1024 vectors, one pass of sources and
// HYBRID_WG_TOKENS < M <= HYBRID_MAX_TOKENS.  (Beyond, kernel W alone wins:
// M = 384, N = 12: 19.25 against 19.58 us in half rows.)
constexpr int HYBRID_WG_TOKENS = 256;
constexpr int HYBRID_MAX_TOKENS = 352;
constexpr int HYBRID_HALF_ROW = 8; // attnres_set_variant(3, 8): half-row chunks

struct Plan {
    int variant = 0; // 1 = workgroup per token, 2 = split hidden, 3 = hybrid
    int vpt = 0;     // 16-byte vectors per thread
    int threads = 0; // threads per workgroup
    int chunks = 1;  // workgroups per token (split part)
    int64_t grid = 0;
    bool single_group = false; // kernel W: all sources of a pass in one group
    int64_t split_base = 0;    // first token of the split part (hybrid: tokens before it are W's)
    int split_threads = 0;     // threads per split chunk
    int wg_blocks = 0;         // hybrid: workgroups of the W part
    int64_t split_slots = 0;   // scratch token slots the call uses (0: no scratch)
};

// Full validation of a fused call; returns a status code (ATTNRES_*).
// out_mix may be NULL (no mixture output).
int validate_fwd(const void* prefix, const void* add, const void* add2, const void* const* snapshots,
                 int n, const void* query, const void* gamma, float eps, int64_t M, int64_t H,
                 const void* out_prefix, const void* out_norm, const void* out_mix = nullptr);

// Size-only validation (what attnres_plan checks).
int validate_sizes(int64_t M, int n, int64_t H);

// Dispatch for (M, N, H).  Never depends on whether add2 is given.
// force_variant / force_param: 0 = automatic, else as attnres_set_variant.
int make_plan(int64_t M, int n, int64_t H, int force_variant, int force_param, Plan& pl);

// Is (variant, param) an accepted dispatch override?
bool valid_override(int variant, int param);

// Validation of the standalone add.
int validate_add(const void* a, const void* b, const void* out, int64_t n);

} // namespace attnres
