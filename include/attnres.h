/*
 * libattnres: the fused attention-residual (AttnRes) combine + RMSNorm of one
 * decode step, with the MoE-tail additions folded in, for MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes; every tensor is bf16 (bit patterns held in
 * 16-bit words), row-major and contiguous.  Device pointers must be memory the
 * GPU can read/write (hipMalloc'd or equivalent); host pointers are marked.
 *
 * Operation (per token m, all tokens independent):
 *   1. fold-add     t  = bf16(add + add2)  (t = add when add2 is NULL)
 *                   p' = bf16(prefix + t)
 *      Each addition is a binary32 round-to-nearest-even add of the exactly
 *      widened bf16 values, subnormals kept; the result is rounded to bf16
 *      (nearest even).  p' is written to out_prefix and is bit-for-bit what
 *      two separate bf16 tensor additions produce.  Source: page
 *      "[#20545][perf] Kimi K3: fold the MoE-tail additions into the next
 *      attention-residual" (TensorRT-LLM #20546), sections "Description" and
 *      "Op".
 *   2. mix          sources k_0..k_{N-1} = the N snapshot rows, k_N = p';
 *                   z_s = sum_h q_h * k_{s,h} / sqrt(mean_h(k_{s,h}^2) + eps)
 *                   alpha = softmax(z);   x = sum_s alpha_s * k_s
 *      The page names this step "attention-residual" and notes (section
 *      "Model") that the capture tap needs the pre-norm mixture x; it prints
 *      no formula.  The reading implemented: weightless key RMSNorm, no
 *      temperature, raw (not normalised) sources mixed, p' taken after its
 *      bf16 rounding.
 *   3. RMSNorm      out_norm = bf16(x / sqrt(mean_h(x_h^2) + eps) * gamma)
 *      x stays binary32 (never rounded to bf16 before the norm).
 *
 * Accuracy contract: out_prefix is bit-exact; out_norm is within 2 bf16 ulps
 * (or 1e-2 absolute) of the same formula evaluated in binary64 with one final
 * rounding.  Results are deterministic: the same inputs and the same dispatch
 * give the same bits, and the dispatch never depends on whether add2 is given,
 * so add2 = s yields the same bits as add = bf16(add + s), add2 = NULL.
 *
 * Execution: stream-ordered and asynchronous.  The fused calls allocate
 * nothing, never synchronise with the host and print nothing; they may be
 * captured into a HIP graph.  The library's per-device scratch is allocated
 * (synchronously) by attnres_init(), which must run once on a device before
 * the first fused call there.  Every argument is validated before any HIP
 * call; an invalid call launches nothing.
 */
#ifndef ATTNRES_H
#define ATTNRES_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define ATTNRES_OK 0
#define ATTNRES_EINVAL (-1)       /* null required pointer, M < 0 or M > INT32_MAX,
                                     n_snapshots < 0, H not a positive multiple of 8,
                                     H above ATTNRES_MAX_HIDDEN,
                                     pointer not 16-byte aligned, eps < 0 or not finite,
                                     bad variant request */
#define ATTNRES_EUNSUPPORTED (-2) /* n_snapshots > ATTNRES_MAX_SNAPSHOTS: the caller
                                     adds the tail first and takes an unfused route
                                     (the page's fallback beyond its source limit,
                                     section "Model") */
#define ATTNRES_EALIAS (-3)       /* forbidden overlap between an output and any other
                                     buffer */
#define ATTNRES_EHIP (-4)         /* a HIP call failed (launch error, no device,
                                     out of memory for the scratch) */
#define ATTNRES_ENOINIT (-5)      /* a fused call on a device where attnres_init()
                                     has not run: nothing was launched */
#define ATTNRES_ESCRATCH (-6)     /* attnres_add_rmsnorm_fwd_noalloc: the call would
                                     need more token slots than its static scratch
                                     holds (ATTNRES_NOALLOC_MAX_SPLIT_TOKENS): nothing
                                     was launched */

#define ATTNRES_MAX_SNAPSHOTS 64 /* up to 12 (the page's fused window, section "Model")
                                    the sources are taken in one pass; 13..64 are fused
                                    too (the workgroup-per-token kernel carries one
                                    running softmax over batches of 12 snapshots; the
                                    split-hidden kernel, used for a few tokens, holds
                                    up to 31 at once in one wave per chunk and up to 63
                                    in two or four), so the page's N > 12 fallback is
                                    not needed below 65 */
#define ATTNRES_MAX_HIDDEN 16384
#define ATTNRES_NOALLOC_MAX_SPLIT_TOKENS 96 /* token slots of the no-allocation scratch */

/*
 * attnres_add_rmsnorm_fwd -- the fused decode step described above.
 *
 *   prefix       device bf16 [M,H]  running prefix sum (read)
 *   add          device bf16 [M,H]  first addend, e.g. routed MoE output (read)
 *   add2         device bf16 [M,H]  second addend, e.g. shared-expert output, or
 *                                   NULL for the single-addend form (read)
 *   snapshots    HOST array of n_snapshots device pointers, each bf16 [M,H]
 *                (the snapshot bank, read); may be NULL when n_snapshots == 0.
 *                Entries may repeat.  The array is read during the call only.
 *   n_snapshots  N, 0 <= N <= 64; N = 0 mixes the updated prefix alone (weight
 *                1), i.e. plain fold-add + RMSNorm
 *   query        device bf16 [H]    per-layer query of the mix (read)
 *   gamma        device bf16 [H]    RMSNorm weight, applied as y = x*rstd*gamma
 *   eps          finite, >= 0; added to the mean square in both RMSNorms
 *   M            tokens, >= 0.  M = 0 launches nothing and returns ATTNRES_OK
 *                once N, H and eps are valid; the pointers are not examined.
 *   H            hidden size, a multiple of 8, 8 <= H <= ATTNRES_MAX_HIDDEN
 *   out_prefix   device bf16 [M,H]  updated prefix p' (written).  May equal
 *                prefix exactly (in place); any other overlap with an input or
 *                with out_norm is ATTNRES_EALIAS.
 *   out_norm     device bf16 [M,H]  normalised mixture (written); must not
 *                overlap any other buffer.
 *   stream       HIP stream the work is enqueued on (0 = the null stream)
 *
 * All device pointers must be 16-byte aligned.  The caller owns every buffer
 * and must keep it alive until the stream work completes.  The library owns a
 * per-device scratch buffer used by the split-hidden kernel (tagged partial
 * records and one epoch word per token slot, 17 MB; nothing needs clearing
 * between calls, HIP-graph replays included).  attnres_init() allocates it;
 * the call itself never allocates or synchronises, and returns
 * ATTNRES_ENOINIT (launching nothing) on a device where attnres_init() has
 * not run, whatever kernel the sizes would select.  The scratch holds 512
 * token slots, handed out in turn when a call is enqueued (a call takes M
 * slots, or M - 256 for the hybrid's split part; it starts again from slot 0
 * when the rest would not fit): calls enqueued on different streams of one
 * device may run at the same time, as long as fewer than 512 slots are handed
 * out between the enqueue of the earliest call still running and that of the
 * latest.  A call captured into a HIP graph keeps the slots it was given, so
 * replays of one graph must be ordered with respect to each other (replays of
 * different graphs need not be).  The split-hidden kernel's waits for the other workgroups of a
 * token are bounded; a wait that gives up (which a correct run never does:
 * see attnres_debug_timeouts) makes that token's out_norm (and out_mix)
 * elements that depend on it NaN instead of wrong; out_prefix is unaffected.
 * The records such a call leaves behind can match the tags of later calls on
 * the same token slots, so once attnres_debug_timeouts reports a nonzero
 * count, clear the scratch (attnres_debug_reset_scratch) before trusting
 * later results.
 *
 * Returns ATTNRES_OK or one of the negative codes above.
 */
int attnres_add_rmsnorm_fwd(const void* prefix, const void* add, const void* add2,
                            const void* const* snapshots, int n_snapshots,
                            const void* query, const void* gamma, float eps,
                            int64_t M, int64_t H, void* out_prefix, void* out_norm,
                            hipStream_t stream);

/*
 * attnres_add_rmsnorm_mix_fwd -- the same fused step, also writing the
 * pre-norm mixture for a speculative-decoding hidden-state capture tap (the
 * page's section "Model" lists such a layer among the fused path's fallbacks
 * because the tap needs x; with this call it stays on the fused path).
 *
 *   out_mix      device bf16 [M,H] or NULL: x = sum_s alpha_s * k_s rounded
 *                once to bf16 (nearest even), within 2 bf16 ulps (or 1e-2
 *                absolute) of x evaluated in binary64.  Written in the same
 *                launch; must be 16-byte aligned and must not overlap any other
 *                buffer (ATTNRES_EALIAS).  NULL makes the call identical to
 *                attnres_add_rmsnorm_fwd.
 *
 * Every other argument, the accuracy of out_prefix / out_norm (bitwise the
 * same as attnres_add_rmsnorm_fwd's for the same inputs and dispatch), the
 * scratch and the status codes are those of attnres_add_rmsnorm_fwd.
 */
int attnres_add_rmsnorm_mix_fwd(const void* prefix, const void* add, const void* add2,
                                const void* const* snapshots, int n_snapshots,
                                const void* query, const void* gamma, float eps,
                                int64_t M, int64_t H, void* out_prefix, void* out_norm,
                                void* out_mix, hipStream_t stream);

/*
 * attnres_add_rmsnorm_fwd_noalloc -- attnres_add_rmsnorm_fwd for callers that
 * cannot allocate device memory: code under HIP-graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It allocates nothing and needs no
 * attnres_init(): the split-hidden kernel's scratch is a static device array
 * of the library (about 3.2 MB per device, held until the process ends),
 * with ATTNRES_NOALLOC_MAX_SPLIT_TOKENS token slots.
 *
 * Arguments, accuracy, dispatch and results are those of
 * attnres_add_rmsnorm_fwd (the same kernels, bit for bit the same outputs).
 * A call whose sizes give the split-hidden kernel more than
 * ATTNRES_NOALLOC_MAX_SPLIT_TOKENS tokens (only possible through
 * attnres_set_variant: the automatic dispatch splits at most 96) returns
 * ATTNRES_ESCRATCH and launches nothing.  The first call on a device
 * that uses the static scratch looks up its address (hipGetSymbolAddress; no
 * allocation, no synchronisation) and enqueues one kernel on `stream` that
 * clears it, ordered before the call's own kernel; attnres_init(), if called
 * on the device, does both beforehand.  Every call on a device shares that
 * device's array, at the same token slots (they are not handed out in turn):
 * calls on one device must be ordered with respect to each other (same
 * stream, or synchronised); calls that overlap in time race on it.
 *
 * Returns ATTNRES_OK, ATTNRES_ESCRATCH or one of the codes of
 * attnres_add_rmsnorm_fwd other than ATTNRES_ENOINIT.
 */
int attnres_add_rmsnorm_fwd_noalloc(const void* prefix, const void* add, const void* add2,
                                    const void* const* snapshots, int n_snapshots,
                                    const void* query, const void* gamma, float eps,
                                    int64_t M, int64_t H, void* out_prefix, void* out_norm,
                                    hipStream_t stream);

/*
 * attnres_bf16_add -- the unfused MoE-tail addition: out = bf16(a + b)
 * elementwise (binary32 round-to-nearest add, subnormals kept), n elements.
 * This is the standalone kernel the fold replaces (page "[#20545][perf] Kimi
 * K3: fold the MoE-tail additions ...", sections "Description" and
 * "Performance"); it serves the eager chain and the fused-vs-unfused timing.
 *   a, b, out    device bf16 [n], 16-byte aligned; out may equal a or b exactly,
 *                other overlaps are ATTNRES_EALIAS
 *   n            >= 0 elements (any n; n = 0 launches nothing, returns ATTNRES_OK
 *                and does not examine the pointers)
 */
int attnres_bf16_add(const void* a, const void* b, void* out, int64_t n,
                     hipStream_t stream);

/*
 * attnres_init -- allocate and clear the split-hidden scratch on the current
 * device (synchronously: hipMalloc, hipMemset, hipDeviceSynchronize), and
 * look up and clear the static scratch of attnres_add_rmsnorm_fwd_noalloc.
 * Must run once on each device before the first attnres_add_rmsnorm_fwd /
 * _mix_fwd call there (those return ATTNRES_ENOINIT otherwise); later calls
 * return at once.  Not for use during HIP-graph capture.  Thread-safe.
 * Returns ATTNRES_OK or ATTNRES_EHIP.
 */
int attnres_init(void);

/*
 * attnres_plan -- the launch the fused call would make for (M, N, H), without
 * any HIP call.  *variant: 1 = workgroup per token, 2 = split hidden, 3 =
 * hybrid (one workgroup per token for the first 256 tokens, split-hidden
 * chunks for the rest, in one launch); *chunks: workgroups per token (of the
 * split part); *threads: threads per workgroup.  Any output
 * pointer may be NULL.  Returns ATTNRES_OK or the status the call would return
 * for these sizes.
 */
int attnres_plan(int64_t M, int n_snapshots, int64_t H, int* variant, int* chunks,
                 int* threads);

/*
 * attnres_set_variant -- process-wide dispatch override for tests and
 * benchmarks: variant 0 = automatic (param 0); 1 = workgroup per token, param =
 * 16-byte vectors per thread (0 automatic, or 1, 2, 4); 2 = split hidden, param
 * = waves per workgroup (0 automatic, or 1, 2, 4..8; with 32..63 snapshots only 0,
 * 1 for the two-wave form on 64-vector chunks, or 4 for the four-wave form on
 * 128-vector chunks); 3 = hybrid, param =
 * waves per split chunk (0 automatic, or 1, 2, 4, or 8 for half rows, the
 * workgroup-per-token width; rows of 4104..8192 elements, at most 12
 * snapshots; below 257 tokens the workgroup-per-token part takes about half
 * of them).  A size the forced
 * variant cannot serve makes the fused call return ATTNRES_EINVAL.  Not thread-safe
 * with concurrent calls.  Returns ATTNRES_OK or ATTNRES_EINVAL.
 */
int attnres_set_variant(int variant, int param);

/*
 * attnres_debug_timeouts -- diagnostic: *out = number of times a split-hidden
 * workgroup gave up waiting at a per-token barrier on the current device since
 * the scratch was created (0 in a correct run).  Synchronous (copies one word
 * to the host).  Returns ATTNRES_OK, ATTNRES_EINVAL (out NULL), ATTNRES_ENOINIT
 * or ATTNRES_EHIP.
 */
int attnres_debug_timeouts(unsigned* out);

/*
 * attnres_debug_set_spin_limit -- diagnostic, for tests of the bounded waits:
 * every later split-hidden launch (process-wide) gives up a wait at a
 * per-token barrier after `limit` re-polls instead of the default (limit = 0
 * restores the default, about 2^20).  A wait that gives up counts a timeout
 * (attnres_debug_timeouts) and takes NaN for every value it did not receive,
 * so each out_norm / out_mix element of the call is then either correct or
 * NaN; the kernel still finishes.  Records a timed-out call leaves behind can
 * match a later call's tags, so clear them with attnres_debug_reset_scratch
 * before trusting results again.  Not thread-safe with concurrent calls.
 * Returns ATTNRES_OK.
 */
int attnres_debug_set_spin_limit(unsigned limit);

/*
 * attnres_debug_set_exchange -- diagnostic, for tests of the split-hidden
 * kernel's exchange: mode 0 (the default) reads the records' L2 copies first
 * (the copy the other workgroups of a token, placed on one XCD, see at once)
 * and their device-scope copies after a bounded number of re-polls; mode 1
 * reads the device-scope copies only; mode 2 reads as mode 0 but places the
 * chunks of a token on different XCDs, so that the L2 copies are not seen and
 * every wait falls back to the device-scope copies.  Outputs are the same bits
 * in every mode; modes 1 and 2 are slower.  Applies to later launches,
 * process-wide.  Not thread-safe with concurrent calls.  Returns ATTNRES_OK
 * or ATTNRES_EINVAL (mode outside 0..2).
 */
int attnres_debug_set_exchange(int mode);

/*
 * attnres_debug_set_slot_rotation -- diagnostic, for tests that need calls on
 * the same token slots of the scratch: on = 0 makes every later call start at
 * slot 0 instead of taking the next slots in turn (on != 0, the default,
 * restores that).  Process-wide; not thread-safe with concurrent calls.
 * Returns ATTNRES_OK.
 */
int attnres_debug_set_slot_rotation(int on);

/*
 * attnres_debug_reset_scratch -- diagnostic: clears the split-hidden scratch of
 * the current device (records, epoch words, timeout counter) synchronously,
 * and hands out token slots from slot 0 again.
 * No call may be in flight on the device.  Not for use during HIP-graph
 * capture.  Returns ATTNRES_OK, ATTNRES_ENOINIT or ATTNRES_EHIP.
 */
int attnres_debug_reset_scratch(void);

/*
 * attnres_debug_set_epoch -- diagnostic, for tests of the split kernel's epoch
 * wrap: sets the epoch word of every token slot of the current device's
 * scratch to `epoch` (synchronously; records are left as they are).  Epochs
 * run through 0 .. 2^31 - 2 and wrap to 0; the call that wraps clears the
 * records of the chunk indices it does not use.  No call may be in flight on
 * the device.  Returns ATTNRES_OK, ATTNRES_EINVAL (epoch out of range),
 * ATTNRES_ENOINIT or ATTNRES_EHIP.
 */
int attnres_debug_set_epoch(unsigned epoch);

/*
 * attnres_selftest_rounding -- diagnostic: checks on the current device that
 * the packed binary32 -> bf16 conversion the kernels use rounds every one of
 * the 2^32 binary32 inputs to nearest even exactly as rounding by definition
 * does (subnormals and overflow included; NaN must stay NaN).
 * *mismatches = number of inputs that disagree (0 expected).  Synchronous;
 * allocates and frees 16 bytes of device memory.  Returns ATTNRES_OK,
 * ATTNRES_EINVAL (NULL) or ATTNRES_EHIP.
 */
int attnres_selftest_rounding(unsigned long long* mismatches);

/* Human-readable name of a status code (static storage). */
const char* attnres_status_string(int status);

/* Library ABI version: major*10000 + minor*100 + patch. */
int attnres_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_H */
