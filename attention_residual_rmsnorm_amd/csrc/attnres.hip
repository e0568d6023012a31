// libattnres: fused AttnRes combine + RMSNorm with the folded MoE-tail add,
// for gfx950 (MI355X).  C-ABI entry points are declared in include/attnres.h.
//
// Method (page "[#20545][perf] Kimi K3: fold the MoE-tail additions into the
// next attention-residual", sections "Description", "Op", "Model"):
//   A1 fold-add    p' = bf16(prefix + bf16(add + add2))            (bit-exact)
//   A2 partials    per source s: sum_h k_sh^2 and sum_h q_h k_sh
//   A3 softmax     z_s = q.k_s / sqrt(mean(k_s^2) + eps), alpha = softmax(z)
//   A4 combine     x = sum_s alpha_s k_s                (binary32, registers)
//   A5 RMSNorm     out = bf16(x / sqrt(mean(x^2) + eps) * gamma)
// Sources are the N snapshot rows then p'.  The page names the mix but prints
// no formula; the reading implemented is the one stated in include/attnres.h.
//
// Two kernels, both HBM-bound streaming kernels (no dense contraction, so no
// MFMA):
//   W  one workgroup per token: the sources (VPT 16-byte vectors per thread,
//      in registers) are loaded in a software pipeline, source-major across
//      the waves, and mixed two at a time as they arrive (up to four
//      sources as one group), under a running softmax maximum and sum; each
//      group's partials are summed per wave by a butterfly of lane swaps and
//      DPP permutations, then across the waves by one thread per value.  With short rows (at most 256 threads of one vector) all sources
//      form one group, summed in one round.  No inter-workgroup
//      communication.  Used when there are many tokens, for short rows, and
//      for more than 12 sources (in batches of 12).
//   S  split hidden: C workgroups per token, each owning a contiguous chunk of
//      the row (one 16-byte vector per thread).  All chunks of a token are
//      placed on one XCD (workgroup id mod 8).  The 2(N+1) partials and the
//      chunk's share of sum x^2 are exchanged through tagged 64-bit records
//      with relaxed atomics (no fences), each record in two copies: one in
//      the XCD's L2, read first, and a device-scope one, the fallback; with
//      at most six sources the chunk's Gram matrix travels instead and one
//      exchange gives both.  Spreads a few tokens over many CUs, which is
//      what the latency-bound small-M calls need.  Token slots of the
//      scratch are handed out per call.
//   W and S in one launch (the hybrid) just past the CU count.
// Outputs are written with the non-temporal hint in both kernels; kernel W
// writes out_prefix after the token's last group, right before out_norm.
// Both reduce in a fixed order: the same inputs give the same bits, and the
// add2 / no-add2 instantiations share every line after A1.
#include "attnres.h"
#include "attnres_device.hpp"
#include "attnres_host.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <utility>

namespace attnres {

constexpr int REC_STRIDE = 64;           // records per (token, chunk) of the first exchange (>= 2*32)
// Each record has two copies (see publish): per (token, chunk), the first
// exchange's L2 copies are records [0, REC_STRIDE) and the device-scope copies
// [REC_STRIDE, 2 REC_STRIDE); per token, the second exchange's are [0,
// MAX_CHUNKS) and [MAX_CHUNKS, 2 MAX_CHUNKS).
constexpr int REC1_CHUNK = 2 * REC_STRIDE;
constexpr int REC2_SLOT = 2 * MAX_CHUNKS;
// re-polls of a record's L2 copy before its device-scope copy is read instead
constexpr unsigned L2_POLLS = 64;
constexpr int STATE_STRIDE = 32;         // epoch word per token: one 128-byte line each
constexpr unsigned SPIN_LIMIT = 1u << 20;
// Kernel S with at most GRAM_MAX_SOURCES sources (attnres_host.hpp) takes one
// exchange instead of two (the Gram form, see fwd_split).  Its sum of x^2,
// alpha' G alpha, is used when GRAM_COND * (sum x^2 / H + eps) >=
// (sum_s alpha_s |k_s|)^2 / H: then the rounding of G's entries, at most a few
// binary32 ulps of |k_s||k_t| each, moves sum x^2 / H + eps by no more than
// about GRAM_COND such ulps relative; when the sources cancel more than that,
// the second exchange runs instead.
constexpr float GRAM_COND = 64.f;
static_assert(GRAM_MAX_SOURCES + GRAM_MAX_SOURCES * (GRAM_MAX_SOURCES + 1) / 2 <= REC_STRIDE,
              "the Gram form's first exchange: one record per value");

struct Params {
    const uint4* prefix;
    const uint4* add;
    const uint4* add2;
    const uint4* snap[MAX_SPLIT_SNAP]; // snapshot rows (kernel W reads the first MAX_SNAP)
    const uint4* query;
    const uint4* gamma;
    uint4* out_prefix;
    uint4* out_norm;
    uint4* out_mix;     // or null: no pre-norm mixture output
    float eps;
    float inv_h;        // 1/H: mean = sum * inv_h
    int nvec;           // H / 8 (16-byte vectors per row)
    int chunks;         // split hidden: workgroups per token
    int64_t M;
    int64_t split_base;       // split hidden: first token it serves (the hybrid's W part takes [0, split_base))
    int64_t slot_base;        // split hidden: scratch token slot of token split_base
    int split_threads;        // split hidden: threads per chunk (the workgroup's others exit at once)
    int wg_blocks;            // hybrid: workgroups of its W part
    unsigned long long* rec1; // split hidden: [token slot][MAX_CHUNKS][REC1_CHUNK] tagged A2 partials
    unsigned long long* rec2; // split hidden: [token][REC2_SLOT] tagged chunk sums of x^2
    unsigned* state;          // split hidden: [token][STATE_STRIDE] epoch word (index 0)
    unsigned* timeouts;       // split hidden: exchange waits that gave up
    unsigned spin_limit;
    unsigned l2_polls;        // split hidden: re-polls of the L2 copies (0: device-scope copies only)
    int xcd_skew;             // split hidden: 1 places a token's chunks on different XCDs (tests only)
};

// A 16-byte load with the non-temporal hint, for the [M,H] streams: a decode
// step reads each of them once, and between two calls of the op the layer in
// between streams far more than the caches hold, so keeping these lines would
// only displace others.  query and gamma, read by every token of the call, are
// loaded normally.
__device__ __forceinline__ uint4 load_stream(const uint4* p)
{
    uint4 r;
    r.x = __builtin_nontemporal_load(&p->x);
    r.y = __builtin_nontemporal_load(&p->y);
    r.z = __builtin_nontemporal_load(&p->z);
    r.w = __builtin_nontemporal_load(&p->w);
    return r;
}

// Output rows are written once and not read again by this call: streamed with
// the non-temporal hint, so the call does not end with them dirty in L2 (at
// M = 256, N = 1: 6.70 -> 5.98 us per call).
__device__ __forceinline__ void store_stream(uint4* p, const uint4& v)
{
    __builtin_nontemporal_store(v.x, &p->x);
    __builtin_nontemporal_store(v.y, &p->y);
    __builtin_nontemporal_store(v.z, &p->z);
    __builtin_nontemporal_store(v.w, &p->w);
}

// Kernel W's out_prefix is held in registers and written after the token's
// last group is mixed, just before A5, next to out_norm: the [M,H] rows of a
// call are then written in one burst at the end of each token instead of in
// the middle of its read stream.  Written early (non-temporal, or plain from
// nine sources on) the 25-layer M = 256 chain took 9.92 us per launch; written
// late, 9.20 (bench.py's chain: 4,467 -> 4,830 GB/s).  Reads and writes
// interleaved on the same HBM channels cost far more than their bytes.

// Loads of vector v of one token's rows (16 bytes = 8 bf16 each).  The loads
// are unconditional: a lane past the end of the row reads the row's last
// vector again (a valid address).  Its values are never stored, and its
// shares of the sums are dropped (see source_partials and combine), so no
// branch or mask sits between the loads: every load of the thread is in
// flight at once.
template <int NS, bool ADD2, int S, int VPT>
__device__ __forceinline__ void load_vectors(const Params& p, int64_t row, int v, bool ok, uint4& a,
                                             uint4& b, uint4& c, uint4 (&k)[S][VPT], int j, uint4& q,
                                             uint4& g)
{
    const int vc = ok ? v : p.nvec - 1;
    a = load_stream(&p.prefix[row + vc]);
    b = load_stream(&p.add[row + vc]);
    c = ADD2 ? load_stream(&p.add2[row + vc]) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int s = 0; s < NS; ++s)
        k[s][j] = load_stream(&p.snap[s][row + vc]);
    q = p.query[vc];
    g = p.gamma[vc];
}

// Register fence: the compiler must assume the packed sources changed, so it
// widens them again in A4 instead of keeping the widened binary32 copies of A2
// alive across the reduction (which would double the register footprint).
template <int S, int VPT>
__device__ __forceinline__ void fence_sources(uint4 (&k)[S][VPT])
{
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int j = 0; j < VPT; ++j)
            asm volatile("" : "+v"(k[s][j].x), "+v"(k[s][j].y), "+v"(k[s][j].z), "+v"(k[s][j].w));
}

// A1 for VPT vectors: k_new = bf16(prefix + bf16(add + add2)).
template <bool ADD2, int VPT>
__device__ __forceinline__ void fold_add(const uint4* a, const uint4* b, const uint4* c, uint4* out)
{
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const uint4 t = ADD2 ? add_bf16x8(b[j], c[j]) : b[j];
        out[j] = add_bf16x8(a[j], t);
    }
}

// A2 for one source and one thread: sum k^2 and q.k over the thread's VPT
// vectors in a fixed order (vector by vector, pair by pair, on
// v_dot2_f32_bf16); vectors outside the row (ok[j] false) contribute zero.
template <int VPT>
__device__ __forceinline__ float2 source_partial(const uint4 (&x)[VPT], const uint4* q, const bool* ok)
{
    float ss = 0.f, qd = 0.f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        float ssj = dot2_bf16(x[j].x, x[j].x, 0.f);
        ssj = dot2_bf16(x[j].y, x[j].y, ssj);
        ssj = dot2_bf16(x[j].z, x[j].z, ssj);
        ssj = dot2_bf16(x[j].w, x[j].w, ssj);
        float qdj = dot2_bf16(q[j].x, x[j].x, 0.f);
        qdj = dot2_bf16(q[j].y, x[j].y, qdj);
        qdj = dot2_bf16(q[j].z, x[j].z, qdj);
        qdj = dot2_bf16(q[j].w, x[j].w, qdj);
        ss += ok[j] ? ssj : 0.f;
        qd += ok[j] ? qdj : 0.f;
    }
    return make_float2(ss, qd);
}

// Position of G_st (s <= t) among the S(S+1)/2 entries of the upper triangle
// of the Gram matrix, row by row.
__host__ __device__ constexpr int gram_index(int s, int t, int S) { return s * S - s * (s - 1) / 2 + (t - s); }

// A2 of kernel S's Gram form: part[s] = q.k_s for s < S and
// part[S + gram_index(s, t)] = k_s.k_t for s <= t (the diagonal is sum k_s^2,
// summed in the same order as source_partial's).
template <int S>
__device__ __forceinline__ void gram_partials(const uint4 (&k)[S][1], const uint4* q, const bool* ok, float* part)
{
#pragma unroll
    for (int s = 0; s < S; ++s) {
        float qd = dot2_bf16(q[0].x, k[s][0].x, 0.f);
        qd = dot2_bf16(q[0].y, k[s][0].y, qd);
        qd = dot2_bf16(q[0].z, k[s][0].z, qd);
        qd = dot2_bf16(q[0].w, k[s][0].w, qd);
        part[s] = ok[0] ? qd : 0.f;
#pragma unroll
        for (int t = s; t < S; ++t) {
            float g = dot2_bf16(k[s][0].x, k[t][0].x, 0.f);
            g = dot2_bf16(k[s][0].y, k[t][0].y, g);
            g = dot2_bf16(k[s][0].z, k[t][0].z, g);
            g = dot2_bf16(k[s][0].w, k[t][0].w, g);
            part[S + gram_index(s, t, S)] = ok[0] ? g : 0.f;
        }
    }
}

// A2 for every source: part[2s] = sum k_s^2, part[2s+1] = q.k_s.
template <int S, int VPT>
__device__ __forceinline__ void source_partials(const uint4 (&k)[S][VPT], const uint4* q, const bool* ok,
                                                float* part)
{
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float2 v = source_partial<VPT>(k[s], q, ok);
        part[2 * s] = v.x;
        part[2 * s + 1] = v.y;
    }
}

// 32-bit word w (0..3) of a 16-byte vector: elements 2w (low half) and 2w+1.
__device__ __forceinline__ uint32_t word(const uint4& v, int w)
{
    return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}

// A4 for one thread: x = sum_s alpha_s k_s, and the thread's share of sum x^2
// (vectors outside the row contribute zero).  Sources are taken in pairs
// (s, s+1): one byte permute puts element e of both into one word, and
// v_dot2_f32_bf16 adds k_s*a_s + k_s+1*a_s+1 in one instruction.  The
// weights go in as two bf16 parts each (hi = bf16(a), lo = bf16(a - hi)), so
// they keep 16 significant bits; the bf16 products are exact in binary32.  An
// odd last source is added with a binary32 fma.  Fixed order: pairs in
// source order (hi part, then lo part), then the odd source.
template <int S, int VPT>
__device__ __forceinline__ float combine(const uint4 (&k)[S][VPT], const float* alpha, const bool* ok,
                                         float (&x)[VPT][8])
{
    constexpr int NP = S / 2;
    uint32_t wh[NP > 0 ? NP : 1], wl[NP > 0 ? NP : 1];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const float a0 = alpha[2 * p], a1 = alpha[2 * p + 1];
        wh[p] = pack_bf16(a0, a1);
        wl[p] = pack_bf16(a0 - lo_f32(wh[p]), a1 - hi_f32(wh[p]));
    }
    float sx = 0.f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        float sxj = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float x0 = 0.f, x1 = 0.f;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const uint32_t A = word(k[2 * p][j], w), B = word(k[2 * p + 1][j], w);
                const uint32_t e0 = __builtin_amdgcn_perm(B, A, 0x05040100u); // (A.lo, B.lo)
                const uint32_t e1 = __builtin_amdgcn_perm(B, A, 0x07060302u); // (A.hi, B.hi)
                x0 = dot2_bf16(e0, wh[p], x0);
                x0 = dot2_bf16(e0, wl[p], x0);
                x1 = dot2_bf16(e1, wh[p], x1);
                x1 = dot2_bf16(e1, wl[p], x1);
            }
            if (S & 1) {
                const uint32_t A = word(k[S - 1][j], w);
                x0 = __builtin_fmaf(alpha[S - 1], lo_f32(A), x0);
                x1 = __builtin_fmaf(alpha[S - 1], hi_f32(A), x1);
            }
            x[j][2 * w] = x0;
            x[j][2 * w + 1] = x1;
            sxj = __builtin_fmaf(x0, x0, sxj);
            sxj = __builtin_fmaf(x1, x1, sxj);
        }
        sx += ok[j] ? sxj : 0.f;
    }
    return sx;
}

// Eight binary32 values times s, rounded to bf16 and packed.
__device__ __forceinline__ uint4 pack_scaled(const float (&x)[8], float s)
{
    return make_uint4(pack_bf16(x[0] * s, x[1] * s), pack_bf16(x[2] * s, x[3] * s),
                      pack_bf16(x[4] * s, x[5] * s), pack_bf16(x[6] * s, x[7] * s));
}

__device__ __forceinline__ uint4 normalise(const float (&x)[8], float rstd, const uint4& g)
{
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        y[e] = (x[e] * rstd) * elem(g, e);
    return make_uint4(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3]), pack_bf16(y[4], y[5]),
                      pack_bf16(y[6], y[7]));
}

// ---------------------------------------------------------------------------
// Kernel W: one workgroup per token (grid-stride over tokens).  Thread `tid`
// owns vectors tid + j*blockDim.x, j < VPT, of the row (coalesced 16-byte
// loads).  blockDim.x is a multiple of 64, at most MAXB.
//
// The token's sources are p' (from prefix, add, add2) and snapshots 0..N-1,
// consumed in that order in groups of up to G (the last source alone; up to
// ONE_GROUP sources form a single group): A2 for
// the group, its token-wide sums, its logits, and its share of A4 under a
// running maximum and running sum of the softmax (what was gathered so far is
// rescaled when the maximum grows).  Loads are software-pipelined LA groups
// ahead: the loads of group g + LA are issued, then group g is mixed, so each
// group's work runs while later groups are in flight and after the last load
// lands only one source's step and A5 remain.  (A CU accepts loads only as
// fast as memory drains them: a wave that issued all of its loads before any
// work would sit in the issue phase for most of the load time.)
// With VPT = 2 (hidden sizes up to 8192) the kernel is held to 128 VGPRs, so
// two workgroups share a CU once there are more tokens than CUs: the second
// token's loads then overlap the first one's reduction and tail.

// Issue-order fence across the workgroup's waves: a bare s_barrier (no
// memory fence, no wait on outstanding loads).  A CU accepts loads only as
// fast as memory drains them, and each SIMD keeps issuing from its oldest
// wave, so without it a SIMD's first wave would issue all of its sources
// before its second wave issued one: the data would arrive wave by wave and
// no source group would be complete until late.  With a fence after each
// source every wave issues source s before any issues source s + 1, so the
// sources arrive in order across the workgroup and each group can be mixed
// while the next is in flight.
__device__ __forceinline__ void issue_fence()
{
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

// Base address of a token's row, held in scalar registers as one opaque
// value: otherwise the compiler re-splits it into (tensor + thread offset),
// hoisted per source out of the token loop at two VGPRs each, plus the row.
// A load is then this base plus the thread's one 32-bit byte offset.  The
// pointer is typed in the global address space: the opaque value hides where
// it came from, and a generic pointer would turn every load into a flat load,
// which also counts against the LDS counter and so serialises with LDS work.
typedef const __attribute__((address_space(1))) char* gptr_t;
typedef const __attribute__((address_space(1))) uint32_t* gword_t;

__device__ __forceinline__ gptr_t row_base(const uint4* tensor, int64_t row)
{
    gptr_t b = (gptr_t)(const void*)(tensor + row); // generic -> global: same address
    asm volatile("" : "+s"(b));
    return b;
}

__device__ __forceinline__ uint4 load_row(gptr_t base, unsigned byte_off)
{
    const gword_t w = reinterpret_cast<gword_t>(base + byte_off);
    uint4 r;
    r.x = __builtin_nontemporal_load(w + 0);
    r.y = __builtin_nontemporal_load(w + 1);
    r.z = __builtin_nontemporal_load(w + 2);
    r.w = __builtin_nontemporal_load(w + 3);
    return r;
}

// Loads of sources [S0, S1) of a batch, one issue_fence after each source.
// With HASP the batch starts with p' (source 0: prefix, add, add2) and source
// s >= 1 is snap[s - 1]; otherwise source s is snap[s].
template <int S0, int S1, bool HASP, bool ADD2, int VPT, int NK>
__device__ __forceinline__ void issue_range(const Params& p, const uint4* const* snap, int64_t row,
                                            const int (&vc)[VPT], uint4 (&a)[VPT], uint4 (&b)[VPT],
                                            uint4 (&c)[VPT], uint4 (&k)[NK][VPT])
{
    if constexpr (S0 < S1) {
        if constexpr (HASP && S0 == 0) {
            gptr_t pa = row_base(p.prefix, row);
            gptr_t pb = row_base(p.add, row);
            gptr_t pc = ADD2 ? row_base(p.add2, row) : nullptr;
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const unsigned off = (unsigned)vc[j] * 16u;
                a[j] = load_row(pa, off);
                b[j] = load_row(pb, off);
                c[j] = ADD2 ? load_row(pc, off) : make_uint4(0u, 0u, 0u, 0u);
            }
        } else {
            gptr_t src = row_base(snap[HASP ? S0 - 1 : S0], row);
#pragma unroll
            for (int j = 0; j < VPT; ++j)
                k[S0][j] = load_row(src, (unsigned)vc[j] * 16u);
        }
        issue_fence();
        issue_range<S0 + 1, S1, HASP, ADD2, VPT, NK>(p, snap, row, vc, a, b, c, k);
    }
}

__device__ __forceinline__ float uniform(float v)
{
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// 1/sqrt(v) on v_rsq_f32 (about 1 ulp) for v >= eps > 0: never a denormal
// argument, so the library's rescaling around it is not needed.
__device__ __forceinline__ float rsq(float v) { return __builtin_amdgcn_rsqf(v); }

// Workgroup totals of NV <= 8 per-thread values in two levels.  Each wave
// sums its values by the butterfly of wave_totals (value v ends in lane
// v * 64 / V) and those lanes store them at rows[8 * wave + v]; after a
// barrier thread v < NV adds the present waves' entries in wave order (all
// MAXW read at once, those of absent waves dropped by a select, never added)
// and stores tot[v].  After a second barrier every thread reads the same bits.
template <int NV, int MAXW>
__device__ __forceinline__ void group_sums(const float (&part)[NV], float* rows, float* tot, int tid,
                                           int nthreads)
{
    static_assert(NV >= 1 && NV <= 8 && MAXW >= 1 && MAXW <= 16, "at most 8 values and 16 waves");
    const int lane = tid & 63, wave = tid >> 6;
    const float wt = wave_totals<NV>(part, lane);
    const int v = bfly_index<pow2_at_least(NV)>(lane);
    if (v >= 0 && v < NV)
        rows[8 * wave + v] = wt;
    __syncthreads();
    if (tid < NV) {
        const int nw = nthreads >> 6;
        float t[MAXW];
#pragma unroll
        for (int r = 0; r < MAXW; ++r)
            t[r] = rows[8 * r + tid];
        float acc = t[0];
#pragma unroll
        for (int r = 1; r < MAXW; ++r)
            acc = r < nw ? acc + t[r] : acc;
        tot[tid] = acc;
    }
    __syncthreads();
}

// Workgroup totals of NV <= 32 per-thread values, for workgroups of at most
// MAXW waves: each wave sums its values by the butterfly of wave_totals and
// the lanes holding the totals store them at rows[32 * wave + v]; after a
// barrier thread v < NV adds value v over the present waves in order (all
// MAXW entries read at once, those of absent waves dropped by a select, never
// added) and stores tot[v].  After a second barrier every thread reads the
// same bits.  One round for all of a token's sources where the rows are short
// (few threads per token).
template <int NV, int MAXW>
__device__ __forceinline__ void group_sums_wide(const float (&part)[NV], float* rows, float* tot, int tid,
                                                int nthreads)
{
    static_assert(NV >= 1 && NV <= 32, "at most 32 values per group");
    const int lane = tid & 63, wave = tid >> 6;
    const float wt = wave_totals<NV>(part, lane);
    const int v = bfly_index<pow2_at_least(NV)>(lane);
    if (v >= 0 && v < NV)
        rows[32 * wave + v] = wt;
    __syncthreads();
    if (tid < NV) {
        const int nw = nthreads >> 6;
        float t[MAXW];
#pragma unroll
        for (int r = 0; r < MAXW; ++r)
            t[r] = rows[32 * r + tid];
        float acc = t[0];
#pragma unroll
        for (int r = 1; r < MAXW; ++r)
            acc = r < nw ? acc + t[r] : acc;
        tot[tid] = acc;
    }
    __syncthreads();
}

// Running softmax state of one token: x = sum_s e^(z_s - m) k_s and
// den = sum_s e^(z_s - m) over the sources so far, m their largest logit.
// z, m and den hold the same bits in every lane (uniform branches).
template <int VPT>
struct Mix {
    float x[VPT][8];
    float m, den;
};

// A2-A4 for one group of n consecutive sources ks[0..n).
template <int n, int VPT, bool FIRST, bool WIDE, int MAXW>
__device__ __forceinline__ void mix_group(const uint4 (*ks)[VPT], const uint4* q, const bool* ok, Mix<VPT>& mx,
                                          float* rows, float* tot, const Params& p, int tid, int nthreads)
{
    float part[2 * n];
#pragma unroll
    for (int s = 0; s < n; ++s) {
        const float2 v = source_partial<VPT>(ks[s], q, ok);
        part[2 * s] = v.x;
        part[2 * s + 1] = v.y;
    }
    if constexpr (WIDE)
        group_sums_wide<2 * n, MAXW>(part, rows, tot, tid, nthreads);
    else
        group_sums<2 * n, MAXW>(part, rows, tot, tid, nthreads);
    float z[n];
#pragma unroll
    for (int s = 0; s < n; ++s)
        z[s] = uniform(rsq(tot[2 * s] * p.inv_h + p.eps) * tot[2 * s + 1]);
    float zmax = z[0];
#pragma unroll
    for (int s = 1; s < n; ++s)
        zmax = fmaxf(zmax, z[s]);
    if (FIRST) {
        mx.m = zmax;
        mx.den = 0.f;
#pragma unroll
        for (int j = 0; j < VPT; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                mx.x[j][e] = 0.f;
    } else if (zmax > mx.m) {
        const float r = __expf(mx.m - zmax);
        mx.den = mx.den * r;
#pragma unroll
        for (int j = 0; j < VPT; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                mx.x[j][e] = mx.x[j][e] * r;
        mx.m = zmax;
    }
    float w[n];
#pragma unroll
    for (int s = 0; s < n; ++s) {
        w[s] = __expf(z[s] - mx.m);
        mx.den = mx.den + w[s];
    }
    // x += sum_s w_s k_s: sources in pairs on v_dot2_f32_bf16 with each weight
    // split into two bf16 parts (hi = bf16(w), lo = bf16(w - hi), 16
    // significant bits; bf16 products are exact in binary32), an odd last
    // source by binary32 fma.  Fixed order.
    constexpr int NP = n / 2;
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
        const uint32_t wh = pack_bf16(w[2 * pp], w[2 * pp + 1]);
        const uint32_t wl = pack_bf16(w[2 * pp] - lo_f32(wh), w[2 * pp + 1] - hi_f32(wh));
#pragma unroll
        for (int j = 0; j < VPT; ++j)
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const uint32_t A = word(ks[2 * pp][j], ww), B = word(ks[2 * pp + 1][j], ww);
                const uint32_t e0 = __builtin_amdgcn_perm(B, A, 0x05040100u); // (A.lo, B.lo)
                const uint32_t e1 = __builtin_amdgcn_perm(B, A, 0x07060302u); // (A.hi, B.hi)
                float x0 = mx.x[j][2 * ww], x1 = mx.x[j][2 * ww + 1];
                x0 = dot2_bf16(e0, wh, x0);
                x0 = dot2_bf16(e0, wl, x0);
                x1 = dot2_bf16(e1, wh, x1);
                x1 = dot2_bf16(e1, wl, x1);
                mx.x[j][2 * ww] = x0;
                mx.x[j][2 * ww + 1] = x1;
            }
    }
    if (n & 1) {
#pragma unroll
        for (int j = 0; j < VPT; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                mx.x[j][e] = __builtin_fmaf(w[n - 1], elem(ks[n - 1][j], e), mx.x[j][e]);
    }
    // materialise x here: otherwise the compiler sinks this work past the next
    // group's wait, out of the window in which loads are in flight
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        asm volatile("" : "+v"(mx.x[j][0]), "+v"(mx.x[j][1]), "+v"(mx.x[j][2]), "+v"(mx.x[j][3]),
                     "+v"(mx.x[j][4]), "+v"(mx.x[j][5]), "+v"(mx.x[j][6]), "+v"(mx.x[j][7]), "+v"(mx.den));
    __builtin_amdgcn_sched_barrier(0);
}

// Groups over S sources: G at a time over sources [0, S-1), then the last
// source alone; up to max(ONE_GROUP, G) sources form a single group (with so
// few, all loads are in flight at once anyway, and one group needs one set of
// workgroup sums instead of two or three: 2-4 % faster at N <= 3).
// group_count is their number, group_start(i) the first source of group i
// (group_start(group_count) = S).
constexpr int ONE_GROUP = 4;

// LDS totals per group slot: 2 per source, up to one pass of sources in one
// group (group_sums_wide, used by the kernels with G > ONE_GROUP).
constexpr int TOT_SLOT = 32;
static_assert(2 * (MAX_SNAP + 1) <= TOT_SLOT, "one pass of sources in one group");

// Kernel W's LDS floats per group slot: 8 values (group_sums) or, with G >
// ONE_GROUP, 32 (group_sums_wide) for each of the MAXB/64 waves.
template <int G, int MAXB>
constexpr int row_slot()
{
    return (G > ONE_GROUP ? 32 : 8) * (MAXB / 64);
}

template <int S, int G>
constexpr bool single_group()
{
    return S <= ONE_GROUP || S <= G;
}

template <int S, int G>
constexpr int group_count()
{
    return single_group<S, G>() ? (S > 0 ? 1 : 0) : 1 + (S - 1 + G - 1) / G;
}

template <int S, int G>
constexpr int group_start(int i)
{
    return single_group<S, G>() ? (i == 0 ? 0 : S)
                                : i < (S - 1 + G - 1) / G ? i * G : (i == (S - 1 + G - 1) / G ? S - 1 : S);
}

// Kernel W's pipeline over one batch of S sources, step GI: issue the loads of
// group GI + LA, then (batch with p', step 0) apply A1, then mix group GI.
// Group gi uses LDS slot gi % 2.  Any reuse of a slot is ordered by the two
// barriers of every group: a thread writes a group's rows
// only after the previous group's second barrier (the threads that add the
// rows have read that group's), and a group's totals are written only after
// its first barrier (every thread has read the previous totals).  FIRSTBATCH: the first
// group starts the running softmax.
template <int S, int G, int LA, int GI, bool HASP, bool FIRSTBATCH, bool ADD2, int VPT, int MAXB>
__device__ __forceinline__ void stream_groups(const Params& p, const uint4* const* snap, int64_t row,
                                              const int (&vc)[VPT], uint4 (&a)[VPT], uint4 (&b)[VPT],
                                              uint4 (&c)[VPT], uint4 (&k)[S][VPT], const uint4* q, const bool* ok,
                                              Mix<VPT>& mx, float (*rows)[row_slot<G, MAXB>()],
                                              float (*tot)[TOT_SLOT], int tid, int nthreads)
{
    constexpr int NG = group_count<S, G>();
    if constexpr (GI < NG) {
        if constexpr (GI + LA < NG)
            issue_range<group_start<S, G>(GI + LA), group_start<S, G>(GI + LA + 1), HASP, ADD2, VPT, S>(
                p, snap, row, vc, a, b, c, k);
        if constexpr (HASP && GI == 0)
            fold_add<ADD2, VPT>(a, b, c, k[0]); // A1 (p' stored after the batch, see stream_batch)
        constexpr int g0 = group_start<S, G>(GI), g1 = group_start<S, G>(GI + 1);
        mix_group<g1 - g0, VPT, FIRSTBATCH && GI == 0, (G > ONE_GROUP), MAXB / 64>(&k[g0], q, ok, mx, rows[GI & 1],
                                                                              tot[GI & 1], p, tid, nthreads);
        stream_groups<S, G, LA, GI + 1, HASP, FIRSTBATCH, ADD2, VPT, MAXB>(p, snap, row, vc, a, b, c, k, q, ok, mx,
                                                                           rows, tot, tid, nthreads);
    }
}

// One batch of S sources through the pipeline: the first LA groups' loads,
// then the steps; a batch that starts with p' then writes out_prefix.
template <int S, int G, int LA, bool HASP, bool FIRSTBATCH, bool ADD2, int VPT, int MAXB>
__device__ __forceinline__ void stream_batch(const Params& p, const uint4* const* snap, int64_t row,
                                             const int (&vc)[VPT], uint4 (&a)[VPT], uint4 (&b)[VPT],
                                             uint4 (&c)[VPT], uint4 (&k)[S][VPT], const uint4* q, const bool* ok,
                                             Mix<VPT>& mx, float (*rows)[row_slot<G, MAXB>()],
                                             float (*tot)[TOT_SLOT], int tid, int nthreads)
{
    constexpr int NG = group_count<S, G>();
    issue_range<0, group_start<S, G>(LA < NG ? LA : NG), HASP, ADD2, VPT, S>(p, snap, row, vc, a, b, c, k);
    stream_groups<S, G, LA, 0, HASP, FIRSTBATCH, ADD2, VPT, MAXB>(p, snap, row, vc, a, b, c, k, q, ok, mx, rows,
                                                                  tot, tid, nthreads);
    if constexpr (HASP) { // out_prefix (p', source 0) once the batch's sources are all in
#pragma unroll
        for (int j = 0; j < VPT; ++j)
            if (ok[j])
                store_stream(&p.out_prefix[row + tid + j * nthreads], k[0][j]);
    }
}

// LDS set-up shared by both forms of kernel W: A5's per-wave sums of absent
// waves stay zero (ordered before use by the barriers of the first group).
template <int MAXW>
__device__ __forceinline__ void wg_prologue(float* red2, int tid, int nthreads)
{
    const int nw = nthreads >> 6;
    if (tid < MAXW && tid >= nw)
        red2[tid] = 0.f;
}

// A5 (and the optional mixture output) of one token from the running softmax
// state.  A4's division by den is folded into the norm: the mixture is x/den,
// so out = x * scale * gamma with
//   scale = 1/(den*sqrt(mean((x/den)^2) + eps)) = 1/sqrt(mean(x^2) + eps*den^2).
template <int VPT, int MAXW>
__device__ __forceinline__ void wg_finish(const Mix<VPT>& mx, const bool* ok, const uint4* g, const Params& p,
                                          int64_t row, float* red2, int tid, int nthreads, bool more)
{
    const int lane = tid & 63, wave = tid >> 6;
    float sx = 0.f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        float sxj = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            sxj = __builtin_fmaf(mx.x[j][e], mx.x[j][e], sxj);
        sx += ok[j] ? sxj : 0.f;
    }
    sx = wave_sum(sx);
    if (lane == 0)
        red2[wave] = sx;
    __syncthreads();
    float ssum = red2[0];
#pragma unroll
    for (int w = 1; w < MAXW; ++w)
        ssum += red2[w];
    const float scale = rsq(ssum * p.inv_h + (p.eps * mx.den) * mx.den);
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        if (ok[j])
            store_stream(&p.out_norm[row + tid + j * nthreads], normalise(mx.x[j], scale, g[j]));
    if (p.out_mix) { // the pre-norm mixture x/den (a uniform branch)
        const float inv = 1.0f / mx.den;
#pragma unroll
        for (int j = 0; j < VPT; ++j)
            if (ok[j])
                store_stream(&p.out_mix[row + tid + j * nthreads], pack_scaled(mx.x[j], inv));
    }
    if (more)
        __syncthreads(); // LDS reuse by the next token (a uniform branch)
}

// Kernel W's body: tokens t0, t0 + stride, ... below tend, one at a time.
template <int NS, bool ADD2, int VPT, int MAXB, int G, int LA>
__device__ __forceinline__ void wg_tokens(const Params& p, int64_t t0, int64_t tend, int64_t stride)
{
    constexpr int S = NS + 1;
    constexpr int MAXW = MAXB / 64;
    static_assert(MAXB / 64 <= 16, "waves of one group slot");
    static_assert(G <= ONE_GROUP || MAXB <= 512, "group_sums_wide: at most 8 waves");
    __shared__ __align__(16) float rows[2][row_slot<G, MAXB>()];
    __shared__ __align__(16) float tot[2][TOT_SLOT];
    __shared__ float red2[MAXW];

    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int nvec = p.nvec;
    wg_prologue<MAXW>(red2, tid, nthreads);

    for (int64_t t = t0; t < tend; t += stride) {
        const int64_t row = t * (int64_t)nvec;
        uint4 k[S][VPT], q[VPT], g[VPT], a[VPT], b[VPT], c[VPT];
        bool ok[VPT];
        int vc[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = tid + j * nthreads;
            ok[j] = v < nvec;
            vc[j] = ok[j] ? v : nvec - 1; // past the row: reread the last vector, never stored
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            q[j] = p.query[vc[j]];
            g[j] = p.gamma[vc[j]];
        }
        // A1 (in step 0), A2-A4
        Mix<VPT> mx;
        stream_batch<S, G, LA, true, true, ADD2, VPT, MAXB>(p, p.snap, row, vc, a, b, c, k, q, ok, mx, rows, tot, tid,
                                                      nthreads);
        // A5
        wg_finish<VPT, MAXW>(mx, ok, g, p, row, red2, tid, nthreads, t + stride < tend);
    }
}

template <int NS, bool ADD2, int VPT, int MAXB, int G, int LA>
__global__ __launch_bounds__(MAXB, (VPT == 2 ? 4 : 1)) void fwd_wg(Params p)
{
    wg_tokens<NS, ADD2, VPT, MAXB, G, LA>(p, blockIdx.x, p.M, gridDim.x);
}

// ---------------------------------------------------------------------------
// Kernel W for more than MAX_SNAP snapshots: the sources come in batches that
// reuse the same registers.  Batch 0 is p' and snapshots 0..MAX_SNAP-1 (the
// code of fwd_wg for N = MAX_SNAP); then pl.n_full batches of MAX_SNAP
// snapshots and a last batch of NB_LAST, each through the same load pipeline
// and mixed into the same running softmax.
struct ParamsLong {
    Params p;
    const uint4* more[MAX_SNAP_LONG - MAX_SNAP]; // snapshots MAX_SNAP, MAX_SNAP + 1, ...
    int n_full;                                  // full batches after batch 0
};

template <int NB_LAST, bool ADD2, int VPT, int MAXB, int G, int LA>
__global__ __launch_bounds__(MAXB, (VPT == 2 ? 4 : 1)) void fwd_wg_long(ParamsLong pl)
{
    constexpr int B = MAX_SNAP;
    constexpr int MAXW = MAXB / 64;
    static_assert(G <= ONE_GROUP || MAXB <= 512, "group_sums_wide: at most 8 waves");
    __shared__ __align__(16) float rows[2][row_slot<G, MAXB>()];
    __shared__ __align__(16) float tot[2][TOT_SLOT];
    __shared__ float red2[MAXW];
    const Params& p = pl.p;

    const int tid = threadIdx.x;
    const int nthreads = blockDim.x;
    const int nvec = p.nvec;
    wg_prologue<MAXW>(red2, tid, nthreads);

    for (int64_t t = blockIdx.x; t < p.M; t += gridDim.x) {
        const int64_t row = t * (int64_t)nvec;
        uint4 q[VPT], g[VPT];
        bool ok[VPT];
        int vc[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = tid + j * nthreads;
            ok[j] = v < nvec;
            vc[j] = ok[j] ? v : nvec - 1;
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            q[j] = p.query[vc[j]];
            g[j] = p.gamma[vc[j]];
        }
        Mix<VPT> mx;
        uint4 a[VPT], b[VPT], c[VPT];
        {
            uint4 k[B + 1][VPT];
            stream_batch<B + 1, G, LA, true, true, ADD2, VPT, MAXB>(p, p.snap, row, vc, a, b, c, k, q, ok, mx, rows, tot,
                                                              tid, nthreads);
        }
        for (int bi = 0; bi < pl.n_full; ++bi) {
            uint4 k[B][VPT];
            stream_batch<B, G, LA, false, false, ADD2, VPT, MAXB>(p, pl.more + bi * B, row, vc, a, b, c, k, q, ok, mx,
                                                            rows, tot, tid, nthreads);
        }
        {
            uint4 k[NB_LAST][VPT];
            stream_batch<NB_LAST, G, LA, false, false, ADD2, VPT, MAXB>(p, pl.more + pl.n_full * B, row, vc, a, b, c, k,
                                                                  q, ok, mx, rows, tot, tid, nthreads);
        }
        wg_finish<VPT, MAXW>(mx, ok, g, p, row, red2, tid, nthreads, t + gridDim.x < p.M);
    }
}

// ---------------------------------------------------------------------------
// The split kernel's per-token epoch.  Epochs run through [0, EPOCH_PERIOD)
// and wrap to 0, so the tags 2E+1 and 2E+2 are never 0, the tag of a record
// that was never written (or was cleared).  A record from an earlier call
// could match a later call's tag only if exactly a multiple of EPOCH_PERIOD
// calls lay between the two, none of which rewrote it.  The call that wraps
// the epoch therefore clears every record it does not read itself: the chunk
// indices it does not use, the first-exchange values past its own count in
// those it does, and the second exchange's records when it has none (the
// Gram form without its fallback).  Only the wrapping call's own records
// survive the wrap, and they could be matched only by the wrapping call of a
// later period if no call of that whole period rewrote them.  The clearing
// runs in chunk 0 after every chunk of its call has read E, touches no record
// any chunk of this call still reads, and the next call on the token slot
// starts after this kernel ends (calls on one device's scratch are ordered).
constexpr unsigned EPOCH_PERIOD = 0x7fffffffu;

__device__ __forceinline__ unsigned long long gave_up(unsigned tag)
{
    return ((unsigned long long)tag << 32) | 0x7fc00000u; // the tag, and a quiet NaN
}

// What one call on a token slot reads: chunk indices c < C with first-exchange
// values [0, nv0); the two-wave form also indices SPLIT_LONG_MAX_CHUNKS + c
// with values [0, nv1); and the second exchange's records c < C unless the
// call had no second exchange.
struct RecordUse {
    int C, nv0, nv1;
    bool rec2;
};

__device__ __noinline__ void clear_unread_records(const Params& p, int64_t slot, RecordUse u)
{
    unsigned long long* rec1 = p.rec1 + (size_t)slot * MAX_CHUNKS * REC1_CHUNK;
    unsigned long long* rec2 = p.rec2 + (size_t)slot * REC2_SLOT;
    for (int c = 0; c < MAX_CHUNKS; ++c) {
        const int page1 = c - SPLIT_LONG_MAX_CHUNKS;
        const int used = c < u.C ? u.nv0 : page1 >= 0 && page1 < u.C ? u.nv1 : 0;
        for (int v = used; v < REC_STRIDE; ++v) { // both copies
            __hip_atomic_store(&rec1[c * REC1_CHUNK + v], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&rec1[c * REC1_CHUNK + REC_STRIDE + v], 0ull, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
        if (c >= u.C || !u.rec2) {
            __hip_atomic_store(&rec2[c], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&rec2[MAX_CHUNKS + c], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__device__ __forceinline__ void advance_epoch(const Params& p, unsigned* state, unsigned epoch, int64_t slot,
                                              RecordUse u)
{
    const unsigned next = epoch + 1u >= EPOCH_PERIOD ? 0u : epoch + 1u;
    if (next == 0u)
        clear_unread_records(p, slot, u);
    __hip_atomic_store(state, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Kernel S: split hidden.  blockDim.x threads per workgroup, one 16-byte vector
// each; C = p.chunks workgroups per token, chunk c owning vectors
// [c*blockDim.x, (c+1)*blockDim.x).  Workgroup b serves token (b/8/C)*8 + b%8,
// chunk (b/8)%C, so every chunk of a token has the same b mod 8, hence the
// same XCD: the dispatcher deals workgroups to the XCDs in turn, so the
// records' L2 copies reach the token's other chunks (Params::xcd_skew, for
// tests only, adds the chunk index to b mod 8 instead, which spreads a
// token's chunks over several XCDs and makes the readers fall back to the
// device-scope copies); grid = 8*C*ceil(M/8) and workgroups past the last
// token exit at once.
//
// Exchanges (see attnres_device.hpp): the call's epoch E is read from the
// token's state word at the start; the A2 partials travel with tag 2E+1, the
// chunk sums of x^2 with tag 2E+2.  Chunk 0 advances the state word (to E+1,
// or to 0 at the end of the period, see advance_epoch) after it has seen
// every chunk's last record, i.e. after every workgroup of the token has read
// E, so all workgroups of one call agree on E, and every call (HIP-graph
// replays included) uses new tags.  Every wait is bounded (Params::spin_limit
// re-polls); a wait that gives up counts a timeout and takes NaN for each
// missing value, so the outputs that depend on it are NaN, never silently
// wrong (out_prefix does not depend on any exchange).
//
// Gram form (S <= GRAM_MAX_SOURCES): the first exchange carries q.k_s and the
// chunk's Gram entries k_s.k_t (s <= t) instead of q.k_s and sum k_s^2.  The
// diagonal gives the logits as before, and sum_h x_h^2 = alpha' G alpha, so
// the second exchange is needed only when that form is ill-conditioned
// (GRAM_COND); every workgroup of the token takes the same decision, from the
// same totals in the same order.
//
// Two families: MAXB = 128 (1-2 waves per workgroup, up to 32 chunks) and
// MAXB = 512 (4-8 waves, at most 8 chunks; capped at 128 VGPRs so that two
// workgroups share a CU).
// Kernel S's body for workgroup b of its part of the grid, nthreads threads
// per chunk (threads beyond exit at once, before any barrier); its tokens are
// split_base + 0, 1, ..., and token slot t - split_base of the scratch serves
// token t.
template <int NS, bool ADD2, int MAXB, int MAXC>
__device__ __forceinline__ void split_chunk(const Params& p, int b, int nthreads)
{
    constexpr int S = NS + 1;
    constexpr bool GRAM = S <= GRAM_MAX_SOURCES;
    constexpr int NV = GRAM ? S + S * (S + 1) / 2 : 2 * S; // values of the first exchange
    constexpr int NVP = (NV + 3) / 4 * 4;
    static_assert(S <= 32 && NV <= 64 && NV <= REC_STRIDE && MAXC <= 64, "one lane per value and per chunk");
    // 1-2 waves per workgroup: every wave gathers the records itself (no
    // barrier after either exchange); 4-8 waves: wave 0 gathers and shares
    // through LDS (less polling traffic when many workgroups wait at once)
    constexpr bool PERWAVE = MAXB <= 128;
    __shared__ __align__(16) float wsum[(MAXB / 64) * NVP];
    __shared__ float red2[MAXB / 64];
    __shared__ float alpha_sh[PERWAVE ? 1 : 32];
    __shared__ float ssum_sh;
    __shared__ float gram_sh[2]; // Gram form, 4-8 waves: wave 0's sum of x^2 and decision

    const int tid = threadIdx.x;
    if (tid >= nthreads)
        return;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nw = nthreads >> 6;
    const int C = p.chunks;
    const int ib = b >> 3;
    const int chunk = ib - (ib / C) * C;
    const int64_t rel = (int64_t)(ib / C) * 8 + ((b + p.xcd_skew * chunk) & 7);
    const int64_t t = p.split_base + rel;
    const int64_t slot = p.slot_base + rel;
    if (t >= p.M)
        return;

    unsigned* state = p.state + (size_t)slot * STATE_STRIDE;
    const unsigned epoch = __hip_atomic_load(state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned tag1 = 2u * epoch + 1u, tag2 = 2u * epoch + 2u;

    const int nvec = p.nvec;
    const int64_t row = t * (int64_t)nvec;
    uint4 k[S][1], q[1], g[1], a[1], bb[1], c[1];
    bool ok[1];
    const int v = chunk * nthreads + tid;
    ok[0] = v < nvec;
    load_vectors<NS, ADD2>(p, row, v, ok[0], a[0], bb[0], c[0], k, 0, q[0], g[0]);
    __builtin_amdgcn_sched_barrier(0);

    // A1
    fold_add<ADD2, 1>(a, bb, c, k[NS]);
    if (ok[0])
        store_stream(&p.out_prefix[row + v], k[NS][0]);

    // A2: this chunk's partials, each wave's totals by the butterfly (one value
    // per lane); one wave publishes them from those lanes, more than one add
    // the waves' totals in order through LDS (thread v < NV: value v)
    float part[NV];
    if constexpr (GRAM)
        gram_partials<S>(k, q, ok, part);
    else
        source_partials<S, 1>(k, q, ok, part);
    fence_sources<S, 1>(k);
    const float wt = wave_totals<NV>(part, lane);
    const int wv = bfly_index<pow2_at_least(NV)>(lane);
    unsigned long long* rec1 = p.rec1 + (size_t)slot * MAX_CHUNKS * REC1_CHUNK;
    if (nw == 1) {
        if (wv >= 0 && wv < NV)
            publish(&rec1[chunk * REC1_CHUNK + wv], REC_STRIDE, tag1, wt);
    } else {
        if (wv >= 0 && wv < NV)
            wsum[wave * NVP + wv] = wt;
        __syncthreads();
        if (tid < NV) {
            float acc = wsum[tid];
            for (int w = 1; w < nw; ++w)
                acc += wsum[w * NVP + tid];
            publish(&rec1[chunk * REC1_CHUNK + tid], REC_STRIDE, tag1, acc);
        }
    }

    // A3 in every wave (PERWAVE) or in wave 0: lane v < NV ends with value v
    // (2s: sum k_s^2, 2s+1: q.k_s) summed over the chunks in a fixed order, up
    // to 16 chunks' records in flight at a time (those not yet tagged read
    // again; bounded wait), so it holds the same bits in every wave of every
    // workgroup of the token.  A
    // DPP swap of neighbouring lanes puts q.k_s beside sum k_s^2 in lane 2s,
    // whose logit, the wave's maximum and the exponentials' sum (DPP and
    // scalar reads, fixed order) give alpha_s in lane 2s.
    float alpha[S];
    float gram_ssum = 0.f; // Gram form: alpha' G alpha
    int use_gram = 0;      // Gram form: 1 when it is well-conditioned (same in every workgroup)
    if (PERWAVE || wave == 0) {
        const unsigned long long ready_zero = (unsigned long long)tag1 << 32; // absent: reads as 0
        // With at most 32 values, lanes v and v + 32 both take value v, from
        // alternate chunks (c0 + h, c0 + h + 2, ...), so 16 chunks' records are
        // in flight at once (one round trip for 14 one-wave chunks instead of
        // two: M = 1, N = 12: 6.32 -> 5.81 us), and the two halves' sums are
        // added at the end (the same bits in both lanes).
        constexpr int HALVES = NV <= 32 ? 2 : 1;
        const int hh = HALVES == 2 ? lane >> 5 : 0;
        const int vv = HALVES == 2 ? lane & 31 : lane;
        float tv = 0.f;
        for (int c0 = 0; c0 < C; c0 += 8 * HALVES) {
            unsigned long long r0[8];
            int off = p.l2_polls ? 0 : REC_STRIDE; // the L2 copies first (see publish)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int cj = c0 + hh + HALVES * j;
                r0[j] = cj < C && vv < NV ? peek(&rec1[cj * REC1_CHUNK + off + vv]) : ready_zero;
            }
            for (unsigned polls = 0;; ++polls) {
                bool ready = true;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    ready &= tag_of(r0[j]) == tag1;
                if (ready)
                    break;
                if (polls >= p.spin_limit) {
                    // give up: a record still missing counts as NaN, so the weights, every
                    // output of this wave and every sum of x^2 it publishes are NaN
                    atomicAdd(p.timeouts, 1u);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (tag_of(r0[j]) != tag1)
                            r0[j] = gave_up(tag1);
                    break;
                }
                if (polls >= p.l2_polls)
                    off = REC_STRIDE; // then the device-scope copies
                __builtin_amdgcn_s_sleep(1);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int cj = c0 + hh + HALVES * j;
                    if (cj < C && vv < NV && tag_of(r0[j]) != tag1)
                        r0[j] = peek(&rec1[cj * REC1_CHUNK + off + vv]);
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                tv += __uint_as_float((unsigned)r0[j]);
        }
        if constexpr (HALVES == 2)
            tv = tv + __shfl_xor(tv, 32);
        float al;
        if constexpr (GRAM) {
            // lane s < S holds q.k_s and fetches G_ss; alpha_s ends in lane s.
            // Lane S + gram_index(s, t) holds G_st and fetches alpha_s, alpha_t.
            const bool src = lane < S;
            const float gss = __shfl(tv, src ? S + gram_index(lane, lane, S) : lane);
            const float z = src ? rsqrtf(gss * p.inv_h + p.eps) * tv : -INFINITY;
            const float zmax = wave_max(z);
            const float e = src ? __expf(z - zmax) : 0.f;
            const float den = wave_sum(e);
            al = e * (1.0f / den);
            int ps = 0, pt = 0, r = lane - S;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                if (r >= 0 && r < S - s) {
                    ps = s;
                    pt = s + r;
                }
                r -= S - s;
            }
            const float as = __shfl(al, ps), at = __shfl(al, pt);
            const bool entry = lane >= S && lane < NV;
            gram_ssum = wave_sum(entry ? ((ps == pt ? 1.f : 2.f) * (as * at)) * tv : 0.f);
            const float cs = wave_sum(src ? al * sqrtf(gss) : 0.f);
            use_gram = GRAM_COND * (gram_ssum * p.inv_h + p.eps) >= (cs * cs) * p.inv_h ? 1 : 0;
            if constexpr (PERWAVE) {
#pragma unroll
                for (int i = 0; i < S; ++i)
                    alpha[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), i));
            } else {
                if (src)
                    alpha_sh[lane] = al;
                if (lane == 0) {
                    gram_sh[0] = gram_ssum;
                    gram_sh[1] = use_gram ? 1.f : 0.f;
                }
            }
        } else {
            const float qd = dpp<0xb1>(tv); // quad_perm [1,0,3,2]: lane 2s gets lane 2s+1's value
            const bool src = (lane & 1) == 0 && lane < NV;
            const float z = src ? rsqrtf(tv * p.inv_h + p.eps) * qd : -INFINITY;
            const float zmax = wave_max(z);
            const float e = src ? __expf(z - zmax) : 0.f;
            const float den = wave_sum(e);
            al = e * (1.0f / den);
            if constexpr (PERWAVE) {
#pragma unroll
                for (int i = 0; i < S; ++i)
                    alpha[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 2 * i));
            } else if (src) {
                alpha_sh[lane >> 1] = al;
            }
        }
    }
    if constexpr (!PERWAVE) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < S; ++i)
            alpha[i] = alpha_sh[i];
        if constexpr (GRAM) {
            gram_ssum = gram_sh[0];
            use_gram = gram_sh[1] != 0.f ? 1 : 0;
        }
    }
    // the same value in every lane and wave of the workgroup: a scalar branch
    use_gram = __builtin_amdgcn_readfirstlane(use_gram);

    // A4
    float x[1][8];
    const float sx = wave_sum(combine<S, 1>(k, alpha, ok, x));
    float ssum = 0.f;
    if (GRAM && use_gram) {
        // A5 from alpha' G alpha: no second exchange.  Chunk 0 has seen every
        // chunk's first record, so every workgroup of the token has read E.
        ssum = gram_ssum;
        if (chunk == 0 && tid == 0)
            advance_epoch(p, state, epoch, slot, RecordUse{C, NV, 0, false});
    } else {
        if (lane == 0)
            red2[wave] = sx;
        __syncthreads();

        // A5: the chunk's sum of x^2 (its waves in order) published by thread 0;
        // every wave (PERWAVE) or wave 0 reads the C records (lane c: chunk c) and
        // adds them on DPP
        unsigned long long* rec2 = p.rec2 + (size_t)slot * REC2_SLOT;
        if (tid == 0) {
            float s2 = red2[0];
            for (int w = 1; w < nw; ++w)
                s2 += red2[w];
            publish(&rec2[chunk], MAX_CHUNKS, tag2, s2);
        }
        if (PERWAVE || wave == 0) {
            int off = p.l2_polls ? 0 : MAX_CHUNKS; // the L2 copies first, as above
            unsigned long long w2 = lane < C ? peek(&rec2[off + lane]) : (unsigned long long)tag2 << 32;
            for (unsigned polls = 0; tag_of(w2) != tag2; ++polls) {
                if (polls >= p.spin_limit) {
                    atomicAdd(p.timeouts, 1u); // give up: the sum, hence this wave's outputs, is NaN
                    w2 = gave_up(tag2);
                    break;
                }
                if (polls >= p.l2_polls)
                    off = MAX_CHUNKS;
                __builtin_amdgcn_s_sleep(1);
                w2 = peek(&rec2[off + lane]);
            }
            ssum = wave_sum(__uint_as_float((unsigned)w2));
            if (chunk == 0 && tid == 0) // every chunk has published its second record: all have read the epoch
                advance_epoch(p, state, epoch, slot, RecordUse{C, NV, 0, true});
            if (!PERWAVE && lane == 0)
                ssum_sh = ssum;
        }
        if constexpr (!PERWAVE) {
            __syncthreads();
            ssum = ssum_sh;
        }
    }
    const float rstd = rsqrtf(ssum * p.inv_h + p.eps);
    if (ok[0]) {
        store_stream(&p.out_norm[row + v], normalise(x[0], rstd, g[0]));
        if (p.out_mix) // the pre-norm mixture (the weights sum to one here)
            store_stream(&p.out_mix[row + v], pack_scaled(x[0], 1.0f));
    }
}

template <int NS, bool ADD2, int MAXB, int MAXC, int WPE>
__global__ __launch_bounds__(MAXB, WPE) void fwd_split(Params p)
{
    split_chunk<NS, ADD2, MAXB, MAXC>(p, blockIdx.x, blockDim.x);
}

// ---------------------------------------------------------------------------
// Kernel S's two-wave form, for 32..MAX_SPLIT_LONG_SNAP snapshots (S = N + 1
// sources, more than one wave's registers hold): chunks of 64 vectors, at
// most LONG_PAGE per token, the same token placement, epochs, tags and
// bounded waits as kernel S above, and two waves per chunk that share the
// vectors and split the sources.  Source s is snapshot s for s < N and the
// folded prefix for s = N; wave w holds sources 32w .. 32w + 31 in registers
// (wave 1 also computes A1 and holds the folded prefix apart), so every row
// of the chunk is loaded at once and read once.
//  * A2: each wave's 64 values (sum k_s^2, q.k_s of its sources: values 2s
//    and 2s + 1) are summed over the wave by the butterfly and published in
//    page w: the chunk's own records for wave 0, those of chunk index
//    c + LONG_PAGE for wave 1 (never a chunk of this token, as C <= LONG_PAGE).
//  * A3: each wave gathers its page over the C chunks in a fixed order; the
//    two waves' maxima and sums of exponentials meet in LDS (one barrier).
//  * A4: each wave mixes its sources; wave 1 adds its mixture to wave 0's
//    through LDS (second barrier), and wave 0 runs A5 as kernel S's second
//    exchange does and stores the outputs.
constexpr int LONG_WAVE_SOURCES = 32;
constexpr int LONG_PAGE = SPLIT_LONG_MAX_CHUNKS;
constexpr int LONG_TABLE = 2 * LONG_WAVE_SOURCES; // pointer table entries (snapshots 0..63)
static_assert(2 * (MAX_SPLIT_LONG_SNAP + 1) <= 2 * REC_STRIDE && 2 * LONG_PAGE <= MAX_CHUNKS,
              "two record pages per chunk");
static_assert(MAX_SPLIT_LONG_SNAP + 1 <= LONG_TABLE && MAX_SPLIT_LONG_SNAP >= LONG_WAVE_SOURCES,
              "wave 0: snapshots only; wave 1: the rest and the folded prefix");

struct ParamsSplitLong {
    Params p;
    const uint4* snaps[LONG_TABLE]; // snapshot s < n_snap; entries past it repeat the last snapshot
    int n_snap;
};

template <bool ADD2>
__global__ __launch_bounds__(128, 1) void fwd_split_long(ParamsSplitLong pl)
{
    const Params& p = pl.p;
    __shared__ float zs[2][2];                  // per wave: largest logit, sum of exponentials below it
    __shared__ __align__(16) float xs[8][64];   // wave 1's mixture, element e of lane l at [e][l]

    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int C = p.chunks;
    const int ib = b >> 3;
    const int chunk = ib - (ib / C) * C;
    const int64_t rel = (int64_t)(ib / C) * 8 + ((b + p.xcd_skew * chunk) & 7);
    const int64_t t = p.split_base + rel;
    const int64_t slot = p.slot_base + rel;
    if (t >= p.M)
        return;

    unsigned* state = p.state + (size_t)slot * STATE_STRIDE;
    const unsigned epoch = __hip_atomic_load(state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned tag1 = 2u * epoch + 1u, tag2 = 2u * epoch + 2u;

    const int ns = pl.n_snap;
    const int nv = 2 * (ns + 1); // values of the first exchange
    const int s0 = LONG_WAVE_SOURCES * wave;
    const int nvec = p.nvec;
    const int64_t row = t * (int64_t)nvec;
    const int v = chunk * 64 + lane;
    bool ok[1];
    ok[0] = v < nvec;
    const int vc = ok[0] ? v : nvec - 1;

    // every load of the wave in flight at once: the prefix and addends first
    // (wave 1: its fold and A2 values then need only them; 0.3-0.8 us per
    // call against issuing them last), its snapshots (a slot past the last
    // reads the token-independent q row instead and counts as zero), q, and
    // gamma (wave 0)
    uint4 a1[1], bb1[1], c1[1];
    if (wave == 1) {
        a1[0] = load_stream(&p.prefix[row + vc]);
        bb1[0] = load_stream(&p.add[row + vc]);
        c1[0] = ADD2 ? load_stream(&p.add2[row + vc]) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint4 k[LONG_WAVE_SOURCES][1];
    {
        const uint4* ptr[LONG_WAVE_SOURCES];
#pragma unroll
        for (int j = 0; j < LONG_WAVE_SOURCES; ++j)
            ptr[j] = pl.snaps[s0 + j];
#pragma unroll
        for (int j = 0; j < LONG_WAVE_SOURCES; ++j) {
            const bool real = s0 + j < ns; // the same in every lane
            const uint4 x = load_stream(real ? ptr[j] + row + vc : p.query + vc);
            k[j][0] = real ? x : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    const uint4 q = p.query[vc];
    uint4 g = make_uint4(0u, 0u, 0u, 0u), kp[1] = {make_uint4(0u, 0u, 0u, 0u)};
    unsigned long long* rec1 = p.rec1 + (size_t)slot * MAX_CHUNKS * REC1_CHUNK;
    unsigned long long* page = rec1 + (size_t)(chunk + LONG_PAGE * wave) * REC1_CHUNK;
    if (wave == 0) {
        g = p.gamma[vc];
    } else {
        // A1, and the folded prefix's A2 values (2N, 2N + 1, in page 1)
        fold_add<ADD2, 1>(a1, bb1, c1, kp);
        if (ok[0])
            store_stream(&p.out_prefix[row + v], kp[0]);
        const float2 pp = source_partial<1>(kp, &q, ok);
        const float part[2] = {pp.x, pp.y};
        const float wt = wave_totals<2>(part, lane);
        const int wv = bfly_index<2>(lane);
        if (wv >= 0)
            publish(&page[2 * ns - 64 + wv], REC_STRIDE, tag1, wt);
    }

    // A2 of the wave's snapshots: lane v ends with value 64w + v
    {
        float part[2 * LONG_WAVE_SOURCES];
        source_partials<LONG_WAVE_SOURCES, 1>(k, &q, ok, part);
        fence_sources<LONG_WAVE_SOURCES, 1>(k);
        const float wt = wave_totals<2 * LONG_WAVE_SOURCES>(part, lane);
        if (2 * s0 + lane < 2 * ns)
            publish(&page[lane], REC_STRIDE, tag1, wt);
    }

    // A3: lane 2j of the wave's page holds sum k_s^2 and lane 2j + 1 q.k_s, s = 32w + j
    const bool want = 2 * s0 + lane < nv;
    const unsigned long long ready_zero = (unsigned long long)tag1 << 32; // absent: reads as 0
    float tv = 0.f;
    for (int c0 = 0; c0 < C; c0 += 8) {
        unsigned long long r0[8];
        int off = p.l2_polls ? 0 : REC_STRIDE; // the L2 copies first (see publish)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int cj = c0 + j;
            r0[j] = cj < C && want ? peek(&rec1[(cj + LONG_PAGE * wave) * REC1_CHUNK + off + lane]) : ready_zero;
        }
        for (unsigned polls = 0;; ++polls) {
            bool ready = true;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                ready &= tag_of(r0[j]) == tag1;
            if (ready)
                break;
            if (polls >= p.spin_limit) {
                atomicAdd(p.timeouts, 1u);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (tag_of(r0[j]) != tag1)
                        r0[j] = gave_up(tag1);
                break;
            }
            if (polls >= p.l2_polls)
                off = REC_STRIDE; // then the device-scope copies
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int cj = c0 + j;
                if (cj < C && want && tag_of(r0[j]) != tag1)
                    r0[j] = peek(&rec1[(cj + LONG_PAGE * wave) * REC1_CHUNK + off + lane]);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            tv += __uint_as_float((unsigned)r0[j]);
    }
    const float qd = dpp<0xb1>(tv); // quad_perm [1,0,3,2]: lane 2j gets lane 2j+1's value
    const bool src = (lane & 1) == 0 && want;
    const float z = src ? rsqrtf(tv * p.inv_h + p.eps) * qd : -INFINITY;
    const float zm = wave_max(z);
    const float e = src ? __expf(z - zm) : 0.f;
    const float den = wave_sum(e);
    if (lane == 0) {
        zs[wave][0] = zm;
        zs[wave][1] = den;
    }
    __syncthreads();
    // the same bits in both waves and in every chunk: wave 0's terms first
    const float zmax = fmaxf(zs[0][0], zs[1][0]);
    const float total = zs[0][1] * __expf(zs[0][0] - zmax) + zs[1][1] * __expf(zs[1][0] - zmax);
    const float al = e * (__expf(zm - zmax) / total);
    float alpha[LONG_WAVE_SOURCES];
#pragma unroll
    for (int i = 0; i < LONG_WAVE_SOURCES; ++i)
        alpha[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 2 * i));

    // A4: the wave's snapshots (wave 1's slot of the folded prefix holds zero),
    // then wave 1 adds the folded prefix's term and hands its mixture over
    float x[1][8];
    combine<LONG_WAVE_SOURCES, 1>(k, alpha, ok, x);
    if (wave == 1) {
        const float an = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 2 * (ns - s0)));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t A = word(kp[0], w);
            xs[2 * w][lane] = __builtin_fmaf(an, lo_f32(A), x[0][2 * w]);
            xs[2 * w + 1][lane] = __builtin_fmaf(an, hi_f32(A), x[0][2 * w + 1]);
        }
    }
    __syncthreads();
    if (wave == 1)
        return;
    float sx = 0.f;
#pragma unroll
    for (int e8 = 0; e8 < 8; ++e8) {
        x[0][e8] += xs[e8][lane];
        sx = __builtin_fmaf(x[0][e8], x[0][e8], sx);
    }
    sx = wave_sum(ok[0] ? sx : 0.f);

    // A5: as in kernel S (one wave)
    unsigned long long* rec2 = p.rec2 + (size_t)slot * REC2_SLOT;
    if (lane == 0)
        publish(&rec2[chunk], MAX_CHUNKS, tag2, sx);
    int off = p.l2_polls ? 0 : MAX_CHUNKS;
    unsigned long long w2 = lane < C ? peek(&rec2[off + lane]) : (unsigned long long)tag2 << 32;
    for (unsigned polls = 0; tag_of(w2) != tag2; ++polls) {
        if (polls >= p.spin_limit) {
            atomicAdd(p.timeouts, 1u);
            w2 = gave_up(tag2);
            break;
        }
        if (polls >= p.l2_polls)
            off = MAX_CHUNKS;
        __builtin_amdgcn_s_sleep(1);
        w2 = peek(&rec2[off + lane]);
    }
    const float ssum = wave_sum(__uint_as_float((unsigned)w2));
    if (chunk == 0 && lane == 0) // every chunk has published its second record: all have read the epoch
        advance_epoch(p, state, epoch, slot, RecordUse{C, nv < 64 ? nv : 64, nv > 64 ? nv - 64 : 0, true});
    const float rstd = rsqrtf(ssum * p.inv_h + p.eps);
    if (ok[0]) {
        store_stream(&p.out_norm[row + v], normalise(x[0], rstd, g));
        if (p.out_mix)
            store_stream(&p.out_mix[row + v], pack_scaled(x[0], 1.0f));
    }
}

// ---------------------------------------------------------------------------
// Kernel S's four-wave form, also for 32..MAX_SPLIT_LONG_SNAP snapshots: four
// waves per chunk of 128 vectors (two per lane, vectors c*128 + 64i + lane),
// wave w holding sources 16w .. 16w + 15 (source N, the folded prefix, in
// wave N / 16, which also runs A1), so rows of up to 16384 fit in
// SPLIT_LONG_MAX_CHUNKS chunks.  The record layout is the two-wave form's
// (value g in page g / 64, slot g % 64); each wave publishes and gathers
// its 32 values, lanes l and l + 32 taking value l from alternate chunks, so
// one round of polls covers 16 chunks.  The waves' largest logits and sums
// meet in LDS (one barrier), waves 1..3 hand their mixtures to wave 0 (a
// second), and wave 0 runs A5 and stores.  Wider calls take this form (it
// halves the chunks per token and their polling), small ones the two-wave
// form (its chunks hold half the work).
constexpr int QUAD_SOURCES = 16;
static_assert(4 * QUAD_SOURCES == LONG_TABLE && 2 * QUAD_SOURCES <= 32, "one gather round per wave");

template <bool ADD2>
__global__ __launch_bounds__(256, 1) void fwd_split_quad(ParamsSplitLong pl)
{
    const Params& p = pl.p;
    __shared__ float zs[4][2];                  // per wave: largest logit, sum of exponentials below it
    __shared__ __align__(16) float xs[3][16][64];  // waves 1..3's mixtures, element e of lane l at [e][l]

    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int C = p.chunks;
    const int ib = b >> 3;
    const int chunk = ib - (ib / C) * C;
    const int64_t rel = (int64_t)(ib / C) * 8 + ((b + p.xcd_skew * chunk) & 7);
    const int64_t t = p.split_base + rel;
    const int64_t slot = p.slot_base + rel;
    if (t >= p.M)
        return;

    unsigned* state = p.state + (size_t)slot * STATE_STRIDE;
    const unsigned epoch = __hip_atomic_load(state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned tag1 = 2u * epoch + 1u, tag2 = 2u * epoch + 2u;

    const int ns = pl.n_snap;
    const int nv = 2 * (ns + 1);
    const int s0 = QUAD_SOURCES * wave;
    const int nvec = p.nvec;
    const int64_t row = t * (int64_t)nvec;
    bool ok[2];
    int vc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int v = chunk * 128 + j * 64 + lane;
        ok[j] = v < nvec;
        vc[j] = ok[j] ? v : nvec - 1;
    }
    // the prefix's wave issues the prefix and addends first (see the two-wave form)
    const bool pre = ns / QUAD_SOURCES == wave; // this wave holds the folded prefix (source N)
    uint4 a1[2], bb1[2], c1[2];
    if (pre) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            a1[i] = load_stream(&p.prefix[row + vc[i]]);
            bb1[i] = load_stream(&p.add[row + vc[i]]);
            c1[i] = ADD2 ? load_stream(&p.add2[row + vc[i]]) : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    uint4 k[QUAD_SOURCES][2];
    {
        const uint4* ptr[QUAD_SOURCES];
#pragma unroll
        for (int j = 0; j < QUAD_SOURCES; ++j)
            ptr[j] = pl.snaps[s0 + j];
#pragma unroll
        for (int j = 0; j < QUAD_SOURCES; ++j) {
            const bool real = s0 + j < ns;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 x = load_stream(real ? ptr[j] + row + vc[i] : p.query + vc[i]);
                k[j][i] = real ? x : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    }
    uint4 q[2], g[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
    uint4 kp[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
#pragma unroll
    for (int i = 0; i < 2; ++i)
        q[i] = p.query[vc[i]];
    unsigned long long* rec1 = p.rec1 + (size_t)slot * MAX_CHUNKS * REC1_CHUNK;
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            g[i] = p.gamma[vc[i]];
    }
    if (pre) {
        fold_add<ADD2, 2>(a1, bb1, c1, kp);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            if (ok[i])
                store_stream(&p.out_prefix[row + chunk * 128 + i * 64 + lane], kp[i]);
        const float2 pp = source_partial<2>(kp, q, ok);
        const float part[2] = {pp.x, pp.y};
        const float wt = wave_totals<2>(part, lane);
        const int wv = bfly_index<2>(lane);
        const int gv = 2 * ns + wv;
        if (wv >= 0)
            publish(&rec1[(chunk + LONG_PAGE * (gv >> 6)) * REC1_CHUNK + (gv & 63)], REC_STRIDE, tag1, wt);
    }
    {
        float part[2 * QUAD_SOURCES];
        source_partials<QUAD_SOURCES, 2>(k, q, ok, part);
        fence_sources<QUAD_SOURCES, 2>(k);
        const float wt = wave_totals<2 * QUAD_SOURCES>(part, lane);
        const int wv = bfly_index<2 * QUAD_SOURCES>(lane);
        const int gv = 2 * s0 + wv;
        if (wv >= 0 && gv < 2 * ns)
            publish(&rec1[(chunk + LONG_PAGE * (gv >> 6)) * REC1_CHUNK + (gv & 63)], REC_STRIDE, tag1, wt);
    }

    // A3: lanes l and l + 32 take value 32w + (l & 31) from alternate chunks;
    // lane 2j then holds sum k_s^2 and lane 2j + 1 q.k_s, s = 16w + j
    const int hh = lane >> 5, vv = lane & 31;
    const int mygv = 2 * s0 + vv;
    const bool want = mygv < nv;
    const unsigned long long* src = rec1 + (size_t)LONG_PAGE * (mygv >> 6) * REC1_CHUNK + (mygv & 63);
    const unsigned long long ready_zero = (unsigned long long)tag1 << 32;
    float tv = 0.f;
    for (int c0 = 0; c0 < C; c0 += 16) {
        unsigned long long r0[8];
        int off = p.l2_polls ? 0 : REC_STRIDE;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int cj = c0 + hh + 2 * j;
            r0[j] = cj < C && want ? peek(&src[cj * REC1_CHUNK + off]) : ready_zero;
        }
        for (unsigned polls = 0;; ++polls) {
            bool ready = true;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                ready &= tag_of(r0[j]) == tag1;
            if (ready)
                break;
            if (polls >= p.spin_limit) {
                atomicAdd(p.timeouts, 1u);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (tag_of(r0[j]) != tag1)
                        r0[j] = gave_up(tag1);
                break;
            }
            if (polls >= p.l2_polls)
                off = REC_STRIDE;
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int cj = c0 + hh + 2 * j;
                if (cj < C && want && tag_of(r0[j]) != tag1)
                    r0[j] = peek(&src[cj * REC1_CHUNK + off]);
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            tv += __uint_as_float((unsigned)r0[j]);
    }
    tv = tv + __shfl_xor(tv, 32);
    const float qd = dpp<0xb1>(tv);
    const bool srcl = (lane & 1) == 0 && lane < 32 && want;
    const float z = srcl ? rsqrtf(tv * p.inv_h + p.eps) * qd : -INFINITY;
    const float zm = wave_max(z);
    const float e = srcl ? __expf(z - zm) : 0.f;
    const float den = wave_sum(e);
    if (lane == 0) {
        zs[wave][0] = zm;
        zs[wave][1] = den;
    }
    __syncthreads();
    const float zmax = fmaxf(fmaxf(zs[0][0], zs[1][0]), fmaxf(zs[2][0], zs[3][0]));
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        total += zs[w][1] * __expf(zs[w][0] - zmax);
    const float al = e * (__expf(zm - zmax) / total);
    float alpha[QUAD_SOURCES];
#pragma unroll
    for (int i = 0; i < QUAD_SOURCES; ++i)
        alpha[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 2 * i));

    float x[2][8];
    combine<QUAD_SOURCES, 2>(k, alpha, ok, x);
    if (pre) {
        const float an = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(al), 2 * (ns - s0)));
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t A = word(kp[i], w);
                x[i][2 * w] = __builtin_fmaf(an, lo_f32(A), x[i][2 * w]);
                x[i][2 * w + 1] = __builtin_fmaf(an, hi_f32(A), x[i][2 * w + 1]);
            }
    }
    if (wave != 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e8 = 0; e8 < 8; ++e8)
                xs[wave - 1][8 * i + e8][lane] = x[i][e8];
    }
    __syncthreads();
    if (wave != 0)
        return;
    float sx = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        float sxi = 0.f;
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
            x[i][e8] += xs[0][8 * i + e8][lane];
            x[i][e8] += xs[1][8 * i + e8][lane];
            x[i][e8] += xs[2][8 * i + e8][lane];
            sxi = __builtin_fmaf(x[i][e8], x[i][e8], sxi);
        }
        sx += ok[i] ? sxi : 0.f;
    }
    sx = wave_sum(sx);

    unsigned long long* rec2 = p.rec2 + (size_t)slot * REC2_SLOT;
    if (lane == 0)
        publish(&rec2[chunk], MAX_CHUNKS, tag2, sx);
    int off = p.l2_polls ? 0 : MAX_CHUNKS;
    unsigned long long w2 = lane < C ? peek(&rec2[off + lane]) : (unsigned long long)tag2 << 32;
    for (unsigned polls = 0; tag_of(w2) != tag2; ++polls) {
        if (polls >= p.spin_limit) {
            atomicAdd(p.timeouts, 1u);
            w2 = gave_up(tag2);
            break;
        }
        if (polls >= p.l2_polls)
            off = MAX_CHUNKS;
        __builtin_amdgcn_s_sleep(1);
        w2 = peek(&rec2[off + lane]);
    }
    const float ssum = wave_sum(__uint_as_float((unsigned)w2));
    if (chunk == 0 && lane == 0)
        advance_epoch(p, state, epoch, slot, RecordUse{C, nv < 64 ? nv : 64, nv > 64 ? nv - 64 : 0, true});
    const float rstd = rsqrtf(ssum * p.inv_h + p.eps);
#pragma unroll
    for (int i = 0; i < 2; ++i)
        if (ok[i]) {
            const int64_t at = row + chunk * 128 + i * 64 + lane;
            store_stream(&p.out_norm[at], normalise(x[i], rstd, g[i]));
            if (p.out_mix)
                store_stream(&p.out_mix[at], pack_scaled(x[i], 1.0f));
        }
}

// ---------------------------------------------------------------------------
// The standalone bf16 addition (the unfused tail): 16-byte vectors, grid-stride,
// plus a scalar tail of n % 8 elements.
__global__ __launch_bounds__(256) void bf16_add_kernel(const uint4* a, const uint4* b, uint4* out,
                                                       int64_t nvec, const uint16_t* at,
                                                       const uint16_t* bt, uint16_t* ot, int tail)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride)
        out[i] = add_bf16x8(a[i], b[i]);
    if (blockIdx.x == 0 && (int)threadIdx.x < tail)
        ot[threadIdx.x] = (uint16_t)(pack_bf16(lo_f32(at[threadIdx.x]) + lo_f32(bt[threadIdx.x]), 0.f) & 0xffffu);
}

// ---------------------------------------------------------------------------
// Host side.

using Kernel = void (*)(Params);

constexpr int WG_GROUP = 2;     // sources per reduction group in kernel W
constexpr int WG_LOOKAHEAD = 1; // groups whose loads are in flight ahead of the one being mixed
// Kernel W with at most SHORT_WG_THREADS threads of one vector each (H <=
// 2048): a token's rows are short, every load is in flight at once, and the
// time goes to the rounds of workgroup sums, so all sources of a pass form one
// group with one round of group_sums_wide (H = 896, N = 12: 5.69 -> 4.26 us per
// call for one token, 6.53 -> 5.28 for 256, against groups of two).  It holds
// 128 VGPRs, so for large M (see Plan::single_group) the form with groups of
// two, at 62, keeps more waves per CU and wins.
constexpr int WG_SHORT_GROUP = MAX_SNAP + 1;
constexpr int WG_SHORT_LOOKAHEAD = 1;

// ---------------------------------------------------------------------------
// The hybrid launch (H of 4104..8192, a few more tokens than CUs, one pass of
// sources): workgroups [0, wg_blocks) run kernel W on tokens [0, split_base),
// the rest run kernel S's chunks of split_threads threads (1, 2 or 4 waves;
// the workgroup's other waves exit at once) on tokens [split_base, M).  With
// split_base = the CU count each CU holds one W token and about one chunk,
// instead of some CUs holding two whole tokens and the others one.
constexpr int HYBRID_WG_THREADS_MAX = 512;

template <int NS, bool ADD2>
__global__ __launch_bounds__(HYBRID_WG_THREADS_MAX, 4) void fwd_hybrid(Params p)
{
    if ((int)blockIdx.x < p.wg_blocks) // uniform over the workgroup
        wg_tokens<NS, ADD2, 2, HYBRID_WG_THREADS_MAX, WG_GROUP, WG_LOOKAHEAD>(p, blockIdx.x, p.split_base,
                                                                             p.wg_blocks);
    else {
        // the chunks' waves first in their SIMDs' issue order: their exchanges
        // otherwise wait behind the W tokens' streams on the same CUs (M = 304:
        // N = 4 10.59 -> 9.72 us, N = 12 16.24 -> 15.66; M = 320: N = 8 13.76
        // -> 13.28, N = 12 16.84 -> 16.29..16.55)
        __builtin_amdgcn_s_setprio(3);
        split_chunk<NS, ADD2, HYBRID_WG_THREADS_MAX, 8>(p, (int)blockIdx.x - p.wg_blocks, p.split_threads);
    }
}

template <bool A2, int... I>
constexpr std::array<Kernel, sizeof...(I)> hybrid_table(std::integer_sequence<int, I...>)
{
    return {{&fwd_hybrid<I, A2>...}};
}

template <bool A2, int VPT, int MAXB, int G, int LA, int... I>
constexpr std::array<Kernel, sizeof...(I)> wg_table(std::integer_sequence<int, I...>)
{
    return {{&fwd_wg<I, A2, VPT, MAXB, G, LA>...}};
}

template <bool A2, int MAXB, int MAXC, int WPE, int... I>
constexpr std::array<Kernel, sizeof...(I)> split_table(std::integer_sequence<int, I...>)
{
    return {{&fwd_split<I, A2, MAXB, MAXC, WPE>...}};
}

using Seq = std::make_integer_sequence<int, MAX_SNAP + 1>;
using SeqSplitSmall = std::make_integer_sequence<int, MAX_SPLIT_SNAP + 1>;

// [add2][N]
const std::array<Kernel, MAX_SNAP + 1> kWg1[2] = {wg_table<false, 1, 1024, WG_GROUP, WG_LOOKAHEAD>(Seq{}),
                                                  wg_table<true, 1, 1024, WG_GROUP, WG_LOOKAHEAD>(Seq{})};
const std::array<Kernel, MAX_SNAP + 1> kWg1Small[2] = {
    wg_table<false, 1, SHORT_WG_THREADS, WG_SHORT_GROUP, WG_SHORT_LOOKAHEAD>(Seq{}),
    wg_table<true, 1, SHORT_WG_THREADS, WG_SHORT_GROUP, WG_SHORT_LOOKAHEAD>(Seq{})};
const std::array<Kernel, MAX_SNAP + 1> kWg2[2] = {wg_table<false, 2, 512, WG_GROUP, WG_LOOKAHEAD>(Seq{}),
                                                  wg_table<true, 2, 512, WG_GROUP, WG_LOOKAHEAD>(Seq{})};
const std::array<Kernel, MAX_SNAP + 1> kWg4[2] = {wg_table<false, 4, 512, WG_GROUP, WG_LOOKAHEAD>(Seq{}),
                                                  wg_table<true, 4, 512, WG_GROUP, WG_LOOKAHEAD>(Seq{})};
// more than MAX_SNAP snapshots: [add2][size of the last batch - 1]
using KernelLong = void (*)(ParamsLong);

template <bool A2, int VPT, int MAXB, int G, int... I>
constexpr std::array<KernelLong, sizeof...(I)> wg_long_table(std::integer_sequence<int, I...>)
{
    return {{&fwd_wg_long<I + 1, A2, VPT, MAXB, G, WG_LOOKAHEAD>...}};
}

using SeqBatch = std::make_integer_sequence<int, MAX_SNAP>;
const std::array<KernelLong, MAX_SNAP> kWgLong2[2] = {wg_long_table<false, 2, 512, WG_GROUP>(SeqBatch{}),
                                                      wg_long_table<true, 2, 512, WG_GROUP>(SeqBatch{})};
const std::array<KernelLong, MAX_SNAP> kWgLong4[2] = {wg_long_table<false, 4, 512, WG_GROUP>(SeqBatch{}),
                                                      wg_long_table<true, 4, 512, WG_GROUP>(SeqBatch{})};
// split hidden, 1-2 waves per workgroup (up to 32 chunks)
// (up to MAX_SPLIT_SNAP snapshots: the 1-2-wave family has the registers)
const std::array<Kernel, MAX_SPLIT_SNAP + 1> kSpSmall[2] = {
    split_table<false, 128, MAX_CHUNKS, 1>(SeqSplitSmall{}), split_table<true, 128, MAX_CHUNKS, 1>(SeqSplitSmall{})};
// split hidden, 4-8 waves per workgroup (up to 8 chunks), two workgroups per CU
const std::array<Kernel, MAX_SNAP + 1> kSpLarge[2] = {split_table<false, 512, 8, 4>(Seq{}),
                                                      split_table<true, 512, 8, 4>(Seq{})};
// split hidden, two- and four-wave forms (32..MAX_SPLIT_LONG_SNAP snapshots)
using KernelSplitLong = void (*)(ParamsSplitLong);
const KernelSplitLong kSpLong[2] = {&fwd_split_long<false>, &fwd_split_long<true>};
const KernelSplitLong kSpQuad[2] = {&fwd_split_quad<false>, &fwd_split_quad<true>};
// the hybrid of the two
const std::array<Kernel, MAX_SNAP + 1> kHybrid[2] = {hybrid_table<false>(Seq{}), hybrid_table<true>(Seq{})};

struct Scratch {
    int dev = -1;
    void* base = nullptr;
    unsigned long long* rec1 = nullptr;
    unsigned long long* rec2 = nullptr;
    unsigned* state = nullptr;
    unsigned* timeouts = nullptr;
};

constexpr int MAX_DEVICES = 64;
std::mutex g_mutex;                          // serialises attnres_init
Scratch g_scratch[MAX_DEVICES];              // written once per device, under g_mutex
std::atomic<bool> g_ready[MAX_DEVICES];      // published after g_scratch[dev] is complete
int g_force_variant = 0;
// Token slots of the allocated scratch are handed out in turn, per device,
// when a call is enqueued: [base, base + n) with base the device's next free
// slot, or 0 when the call would run past the last slot.  Calls enqueued on
// different streams therefore use different slots unless MAX_SPLIT_TOKENS
// slots were handed out between them, and may run at the same time.
std::atomic<int64_t> g_slot_next[MAX_DEVICES];
std::atomic<bool> g_rotate{true}; // false: every call starts at slot 0 (tests)
unsigned g_spin_limit = SPIN_LIMIT;
unsigned g_l2_polls = L2_POLLS;
int g_xcd_skew = 0;
int g_force_param = 0;

constexpr size_t REC1_BYTES = sizeof(unsigned long long) * MAX_SPLIT_TOKENS * MAX_CHUNKS * REC1_CHUNK;
constexpr size_t REC2_BYTES = sizeof(unsigned long long) * MAX_SPLIT_TOKENS * REC2_SLOT;
constexpr size_t STATE_BYTES = sizeof(unsigned) * MAX_SPLIT_TOKENS * STATE_STRIDE;
constexpr size_t SCRATCH_BYTES = REC1_BYTES + REC2_BYTES + STATE_BYTES + 256;

int current_device(int* dev)
{
    if (hipGetDevice(dev) != hipSuccess || *dev < 0 || *dev >= MAX_DEVICES)
        return ATTNRES_EHIP;
    return ATTNRES_OK;
}

// Allocates and clears the scratch of the current device (once; attnres_init).
int init_scratch()
{
    int dev = 0;
    int rc = current_device(&dev);
    if (rc != ATTNRES_OK)
        return rc;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_ready[dev].load(std::memory_order_acquire))
        return ATTNRES_OK;
    void* base = nullptr;
    if (hipMalloc(&base, SCRATCH_BYTES) != hipSuccess)
        return ATTNRES_EHIP;
    if (hipMemset(base, 0, SCRATCH_BYTES) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        (void)hipFree(base);
        return ATTNRES_EHIP;
    }
    Scratch& s = g_scratch[dev];
    char* c = static_cast<char*>(base);
    s.rec1 = reinterpret_cast<unsigned long long*>(c);
    s.rec2 = reinterpret_cast<unsigned long long*>(c + REC1_BYTES);
    s.state = reinterpret_cast<unsigned*>(c + REC1_BYTES + REC2_BYTES);
    s.timeouts = reinterpret_cast<unsigned*>(c + REC1_BYTES + REC2_BYTES + STATE_BYTES);
    s.base = base;
    s.dev = dev;
    g_ready[dev].store(true, std::memory_order_release);
    return ATTNRES_OK;
}

// The scratch of the current device, or ATTNRES_ENOINIT when attnres_init has
// not run there.  Never allocates, never synchronises.
int64_t take_slots(int dev, int64_t n)
{
    if (!g_rotate.load(std::memory_order_relaxed))
        return 0;
    int64_t cur = g_slot_next[dev].load(std::memory_order_relaxed);
    for (;;) {
        const int64_t base = cur + n > MAX_SPLIT_TOKENS ? 0 : cur;
        if (g_slot_next[dev].compare_exchange_weak(cur, base + n, std::memory_order_relaxed))
            return base;
    }
}

int scratch_for_current_device(Scratch** out)
{
    int dev = 0;
    int rc = current_device(&dev);
    if (rc != ATTNRES_OK)
        return rc;
    if (!g_ready[dev].load(std::memory_order_acquire))
        return ATTNRES_ENOINIT;
    *out = &g_scratch[dev];
    return ATTNRES_OK;
}

// ---------------------------------------------------------------------------
// The scratch of attnres_add_rmsnorm_fwd_noalloc: a file-scope device array,
// so that entry point never allocates.  Same layout as the allocated scratch
// (records [token][MAX_CHUNKS][REC1_CHUNK], [token][REC2_SLOT], epoch words
// [token][STATE_STRIDE], the timeout counter) for STATIC_SPLIT_TOKENS token
// slots: every call the automatic dispatch makes fits (the split kernel takes
// at most SPLIT_WIDE_TOKENS tokens, the hybrid's split part at most
// HYBRID_MAX_TOKENS - HYBRID_WG_TOKENS).  Each device holds its own copy, at
// its own address, for the life of the process.  In host code `scratch` names a host-side stand-in,
// not device memory: host code uses only the address hipGetSymbolAddress
// returns for the current device (g_static below).
constexpr int STATIC_SPLIT_TOKENS = 96;
static_assert(STATIC_SPLIT_TOKENS >= SPLIT_WIDE_TOKENS && STATIC_SPLIT_TOKENS >= SPLIT_MID_TOKENS &&
                  STATIC_SPLIT_TOKENS >= HYBRID_MAX_TOKENS - HYBRID_WG_TOKENS,
              "every automatic plan fits the static scratch");
constexpr size_t STATIC_REC1_BYTES = sizeof(unsigned long long) * STATIC_SPLIT_TOKENS * MAX_CHUNKS * REC1_CHUNK;
constexpr size_t STATIC_REC2_BYTES = sizeof(unsigned long long) * STATIC_SPLIT_TOKENS * REC2_SLOT;
constexpr size_t STATIC_STATE_BYTES = sizeof(unsigned) * STATIC_SPLIT_TOKENS * STATE_STRIDE;
constexpr size_t STATIC_SCRATCH_BYTES = STATIC_REC1_BYTES + STATIC_REC2_BYTES + STATIC_STATE_BYTES + 256;
static_assert(STATIC_SCRATCH_BYTES % 16 == 0, "cleared in 16-byte vectors");

static __device__ __align__(256) unsigned char scratch[STATIC_SCRATCH_BYTES];

std::mutex g_static_mutex;
std::atomic<unsigned char*> g_static[MAX_DEVICES]; // device address of `scratch`, per device

// Clears n 16-byte vectors (the static scratch, once per device, on the
// caller's stream: a kernel rather than a memset, so a HIP graph may hold it).
__global__ __launch_bounds__(256) void clear_vectors(uint4* p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The static scratch of the current device: its address from
// hipGetSymbolAddress (no allocation, no synchronisation), resolved on first
// use on the device or in attnres_init.  On first use the array is also
// cleared on `stream` (ordered before the call's own kernel); `clear` is false
// only from attnres_init, which clears it synchronously instead.
int static_scratch_for_current_device(Scratch* out, hipStream_t stream, bool clear)
{
    int dev = 0;
    int rc = current_device(&dev);
    if (rc != ATTNRES_OK)
        return rc;
    unsigned char* base = g_static[dev].load(std::memory_order_acquire);
    if (!base) {
        std::lock_guard<std::mutex> lock(g_static_mutex);
        base = g_static[dev].load(std::memory_order_acquire);
        if (!base) {
            void* ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
                return ATTNRES_EHIP;
            const int64_t nvec = (int64_t)(STATIC_SCRATCH_BYTES / 16);
            if (clear) {
                uint4* pv = static_cast<uint4*>(ptr);
                void* args[] = {&pv, (void*)&nvec};
                if (hipLaunchKernel(reinterpret_cast<const void*>(&clear_vectors), dim3(256), dim3(256), args, 0,
                                    stream) != hipSuccess)
                    return ATTNRES_EHIP;
            } else if (hipMemset(ptr, 0, STATIC_SCRATCH_BYTES) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
                return ATTNRES_EHIP;
            }
            base = static_cast<unsigned char*>(ptr);
            g_static[dev].store(base, std::memory_order_release);
        }
    }
    out->base = base;
    out->rec1 = reinterpret_cast<unsigned long long*>(base);
    out->rec2 = reinterpret_cast<unsigned long long*>(base + STATIC_REC1_BYTES);
    out->state = reinterpret_cast<unsigned*>(base + STATIC_REC1_BYTES + STATIC_REC2_BYTES);
    out->timeouts = reinterpret_cast<unsigned*>(base + STATIC_REC1_BYTES + STATIC_REC2_BYTES + STATIC_STATE_BYTES);
    return ATTNRES_OK;
}

} // namespace attnres

using namespace attnres;

namespace attnres {

// The fused call.  static_scratch: the split kernel's scratch is the static
// array (attnres_add_rmsnorm_fwd_noalloc: no attnres_init needed, at most
// STATIC_SPLIT_TOKENS token slots); otherwise the allocated one, which
// attnres_init must have set up on the device.
int launch_fwd(const void* prefix, const void* add, const void* add2, const void* const* snapshots,
               int n_snapshots, const void* query, const void* gamma, float eps, int64_t M, int64_t H,
               void* out_prefix, void* out_norm, void* out_mix, hipStream_t stream, bool static_scratch = false)
{
    int rc = validate_fwd(prefix, add, add2, snapshots, n_snapshots, query, gamma, eps, M, H,
                          out_prefix, out_norm, out_mix);
    if (rc != ATTNRES_OK)
        return rc;
    Plan pl;
    rc = make_plan(M, n_snapshots, H, g_force_variant, g_force_param, pl);
    if (rc != ATTNRES_OK)
        return rc;
    if (M == 0)
        return ATTNRES_OK;
    Scratch static_view;
    Scratch* sc = &static_view;
    if (static_scratch) {
        if (pl.split_slots > STATIC_SPLIT_TOKENS)
            return ATTNRES_ESCRATCH;
        rc = pl.split_slots > 0 ? static_scratch_for_current_device(&static_view, stream, true) : ATTNRES_OK;
    } else {
        // every fused call needs attnres_init on its device (whichever kernel
        // the plan picks, so that the rule does not depend on the sizes)
        rc = scratch_for_current_device(&sc);
    }
    if (rc != ATTNRES_OK)
        return rc;

    Params p{};
    p.prefix = static_cast<const uint4*>(prefix);
    p.add = static_cast<const uint4*>(add);
    p.add2 = static_cast<const uint4*>(add2);
    for (int s = 0; s < n_snapshots && s < MAX_SPLIT_SNAP; ++s)
        p.snap[s] = static_cast<const uint4*>(snapshots[s]);
    p.query = static_cast<const uint4*>(query);
    p.gamma = static_cast<const uint4*>(gamma);
    p.out_prefix = static_cast<uint4*>(out_prefix);
    p.out_norm = static_cast<uint4*>(out_norm);
    p.out_mix = static_cast<uint4*>(out_mix);
    p.eps = eps;
    p.inv_h = 1.0f / (float)H;
    p.nvec = (int)(H / 8);
    p.chunks = pl.chunks;
    p.M = M;
    p.split_base = pl.split_base;
    // the static scratch's slots are fixed (one call at a time per device)
    p.slot_base = !static_scratch && pl.split_slots > 0 ? take_slots(sc->dev, pl.split_slots) : 0;
    p.split_threads = pl.variant == 3 ? pl.split_threads : pl.threads;
    p.wg_blocks = pl.wg_blocks;
    p.spin_limit = g_spin_limit;
    p.l2_polls = g_l2_polls;
    p.xcd_skew = g_xcd_skew;

    const int a2 = add2 ? 1 : 0;
    if (pl.variant == 2 || pl.variant == 3) {
        p.rec1 = sc->rec1;
        p.rec2 = sc->rec2;
        p.state = sc->state;
        p.timeouts = sc->timeouts;
    }
    if (n_snapshots > MAX_SPLIT_SNAP && pl.variant == 2) {
        // the split kernel's two-wave form: one table of snapshot pointers,
        // its tail repeating the last snapshot (never read: see fwd_split_long)
        ParamsSplitLong lp{};
        lp.p = p;
        for (int s = 0; s < LONG_TABLE; ++s)
            lp.snaps[s] = static_cast<const uint4*>(snapshots[s < n_snapshots ? s : n_snapshots - 1]);
        lp.n_snap = n_snapshots;
        void* largs[] = {&lp};
        const KernelSplitLong fl = pl.threads == 256 ? kSpQuad[a2] : kSpLong[a2];
        if (hipLaunchKernel(reinterpret_cast<const void*>(fl), dim3((unsigned)pl.grid), dim3(pl.threads),
                            largs, 0, stream) != hipSuccess)
            return ATTNRES_EHIP;
        return ATTNRES_OK;
    }
    if (n_snapshots > MAX_SNAP && pl.variant == 1) {
        // batched sources: batch 0 = p' + snapshots 0..11, then full batches of
        // 12 and a last batch of 1..12
        ParamsLong lp{};
        lp.p = p;
        for (int s = MAX_SNAP; s < n_snapshots; ++s)
            lp.more[s - MAX_SNAP] = static_cast<const uint4*>(snapshots[s]);
        const int rest = n_snapshots - MAX_SNAP;
        const int nb_last = (rest - 1) % MAX_SNAP + 1;
        lp.n_full = (rest - nb_last) / MAX_SNAP;
        KernelLong fl = (pl.vpt == 2 ? kWgLong2 : kWgLong4)[a2][nb_last - 1];
        void* largs[] = {&lp};
        if (hipLaunchKernel(reinterpret_cast<const void*>(fl), dim3((unsigned)pl.grid), dim3(pl.threads), largs,
                            0, stream) != hipSuccess)
            return ATTNRES_EHIP;
        return ATTNRES_OK;
    }
    Kernel fn = nullptr;
    if (pl.variant == 2 || pl.variant == 3) {
        if (pl.variant == 3)
            fn = kHybrid[a2][n_snapshots];
        else
            fn = pl.threads <= 128 ? kSpSmall[a2][n_snapshots] : kSpLarge[a2][n_snapshots];
    } else {
        const auto& wg1 = pl.single_group ? kWg1Small : kWg1;
        fn = (pl.vpt == 1 ? wg1 : pl.vpt == 2 ? kWg2 : kWg4)[a2][n_snapshots];
    }
    void* args[] = {&p};
    if (hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)pl.grid), dim3(pl.threads),
                        args, 0, stream) != hipSuccess)
        return ATTNRES_EHIP;
    return ATTNRES_OK;
}

} // namespace attnres

extern "C" int attnres_add_rmsnorm_fwd(const void* prefix, const void* add, const void* add2,
                                       const void* const* snapshots, int n_snapshots,
                                       const void* query, const void* gamma, float eps, int64_t M,
                                       int64_t H, void* out_prefix, void* out_norm,
                                       hipStream_t stream)
{
    return launch_fwd(prefix, add, add2, snapshots, n_snapshots, query, gamma, eps, M, H, out_prefix,
                      out_norm, nullptr, stream);
}

extern "C" int attnres_add_rmsnorm_mix_fwd(const void* prefix, const void* add, const void* add2,
                                           const void* const* snapshots, int n_snapshots,
                                           const void* query, const void* gamma, float eps, int64_t M,
                                           int64_t H, void* out_prefix, void* out_norm, void* out_mix,
                                           hipStream_t stream)
{
    return launch_fwd(prefix, add, add2, snapshots, n_snapshots, query, gamma, eps, M, H, out_prefix,
                      out_norm, out_mix, stream);
}

extern "C" int attnres_add_rmsnorm_fwd_noalloc(const void* prefix, const void* add, const void* add2,
                                               const void* const* snapshots, int n_snapshots,
                                               const void* query, const void* gamma, float eps, int64_t M,
                                               int64_t H, void* out_prefix, void* out_norm, hipStream_t stream)
{
    return launch_fwd(prefix, add, add2, snapshots, n_snapshots, query, gamma, eps, M, H, out_prefix,
                      out_norm, nullptr, stream, true);
}

extern "C" int attnres_bf16_add(const void* a, const void* b, void* out, int64_t n, hipStream_t stream)
{
    const int rc = validate_add(a, b, out, n);
    if (rc != ATTNRES_OK || n == 0)
        return rc;
    const int64_t nvec = n / 8;
    const int tail = (int)(n % 8);
    int64_t blocks = (nvec + 255) / 256;
    blocks = std::max<int64_t>(1, std::min<int64_t>(blocks, 4096));
    const uint16_t* at = static_cast<const uint16_t*>(a) + nvec * 8;
    const uint16_t* bt = static_cast<const uint16_t*>(b) + nvec * 8;
    uint16_t* ot = static_cast<uint16_t*>(out) + nvec * 8;
    const uint4* av = static_cast<const uint4*>(a);
    const uint4* bv = static_cast<const uint4*>(b);
    uint4* ov = static_cast<uint4*>(out);
    void* args[] = {&av, &bv, &ov, (void*)&nvec, &at, &bt, &ot, (void*)&tail};
    if (hipLaunchKernel(reinterpret_cast<const void*>(&bf16_add_kernel), dim3((unsigned)blocks), dim3(256),
                        args, 0, stream) != hipSuccess)
        return ATTNRES_EHIP;
    return ATTNRES_OK;
}

extern "C" int attnres_init(void)
{
    const int rc = init_scratch();
    if (rc != ATTNRES_OK)
        return rc;
    Scratch view;
    return static_scratch_for_current_device(&view, nullptr, false);
}

extern "C" int attnres_plan(int64_t M, int n_snapshots, int64_t H, int* variant, int* chunks,
                            int* threads)
{
    int rc = validate_sizes(M, n_snapshots, H);
    if (rc != ATTNRES_OK)
        return rc;
    Plan pl;
    rc = make_plan(M, n_snapshots, H, g_force_variant, g_force_param, pl);
    if (rc != ATTNRES_OK)
        return rc;
    if (variant)
        *variant = pl.variant;
    if (chunks)
        *chunks = pl.chunks;
    if (threads)
        *threads = pl.threads;
    return ATTNRES_OK;
}

extern "C" int attnres_set_variant(int variant, int param)
{
    if (!valid_override(variant, param))
        return ATTNRES_EINVAL;
    g_force_variant = variant;
    g_force_param = param;
    return ATTNRES_OK;
}

extern "C" int attnres_debug_timeouts(unsigned* out)
{
    if (!out)
        return ATTNRES_EINVAL;
    Scratch* sc = nullptr;
    const int rc = scratch_for_current_device(&sc);
    if (rc != ATTNRES_OK)
        return rc;
    if (hipMemcpy(out, sc->timeouts, sizeof(unsigned), hipMemcpyDeviceToHost) != hipSuccess)
        return ATTNRES_EHIP;
    return ATTNRES_OK;
}

extern "C" int attnres_debug_set_spin_limit(unsigned limit)
{
    g_spin_limit = limit ? limit : SPIN_LIMIT;
    return ATTNRES_OK;
}

extern "C" int attnres_debug_set_exchange(int mode)
{
    if (mode < 0 || mode > 2)
        return ATTNRES_EINVAL;
    g_l2_polls = mode == 1 ? 0u : L2_POLLS;
    g_xcd_skew = mode == 2 ? 1 : 0;
    return ATTNRES_OK;
}

extern "C" int attnres_debug_reset_scratch(void)
{
    Scratch* sc = nullptr;
    const int rc = scratch_for_current_device(&sc);
    if (rc != ATTNRES_OK)
        return rc;
    if (hipDeviceSynchronize() != hipSuccess || hipMemset(sc->base, 0, SCRATCH_BYTES) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
        return ATTNRES_EHIP;
    g_slot_next[sc->dev].store(0, std::memory_order_relaxed);
    return ATTNRES_OK;
}

extern "C" int attnres_debug_set_slot_rotation(int on)
{
    g_rotate.store(on != 0, std::memory_order_relaxed);
    return ATTNRES_OK;
}

extern "C" int attnres_debug_set_epoch(unsigned epoch)
{
    if (epoch >= EPOCH_PERIOD)
        return ATTNRES_EINVAL;
    Scratch* sc = nullptr;
    const int rc = scratch_for_current_device(&sc);
    if (rc != ATTNRES_OK)
        return rc;
    static unsigned words[MAX_SPLIT_TOKENS * STATE_STRIDE];
    std::lock_guard<std::mutex> lock(g_mutex);
    for (int t = 0; t < MAX_SPLIT_TOKENS; ++t)
        for (int i = 0; i < STATE_STRIDE; ++i)
            words[t * STATE_STRIDE + i] = i == 0 ? epoch : 0u;
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(sc->state, words, sizeof(words), hipMemcpyHostToDevice) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
        return ATTNRES_EHIP;
    return ATTNRES_OK;
}

extern "C" const char* attnres_status_string(int status)
{
    switch (status) {
    case ATTNRES_OK: return "ok";
    case ATTNRES_EINVAL: return "invalid argument";
    case ATTNRES_EUNSUPPORTED: return "unsupported (more than 64 snapshots): add first, use the unfused route";
    case ATTNRES_EALIAS: return "forbidden buffer overlap";
    case ATTNRES_EHIP: return "HIP error";
    case ATTNRES_ENOINIT: return "attnres_init() has not run on the current device";
    case ATTNRES_ESCRATCH:
        return "the call needs more than the static scratch holds (split-hidden kernel for more than 96 tokens)";
    default: return "unknown status";
    }
}

extern "C" int attnres_version(void) { return 20000; }
