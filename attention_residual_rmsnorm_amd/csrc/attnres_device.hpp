// Device helpers for the gfx950 AttnRes + RMSNorm kernels: bf16 <-> binary32,
// wave-wide sums on DPP, and the per-token barrier of the split-hidden kernel.
//
// Arithmetic conventions (the whole library is built with -ffp-contract=off and
// IEEE binary32 denormals, so every a*b+c below is written as an explicit fma
// or as two rounded operations on purpose):
//   * widening bf16 -> binary32 is exact (a 16-bit shift or a mask);
//   * narrowing binary32 -> bf16 rounds to nearest, ties to even, keeps
//     subnormals, overflows to +-Inf and keeps NaN quiet (pack_bf16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

// ---- bf16 <-> binary32 --------------------------------------------------

__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element e (0..7) of eight packed bf16 values, widened exactly.
__device__ __forceinline__ float elem(const uint4& v, int e)
{
    const uint32_t w = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
    return (e & 1) ? hi_f32(w) : lo_f32(w);
}

// Two binary32 values rounded to bf16 and packed (lo in bits 15:0).  The
// conversion compiles to gfx950's v_cvt_pk_bf16_f32, which rounds to nearest
// even, keeps subnormals (the kernels run with IEEE binary32 denormals),
// overflows to +-Inf and returns a quiet NaN for NaN; this equals rounding by
// definition on every binary32 input (checked exhaustively on the device by
// attnres_selftest_rounding).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    bf16x2_t r;
    r.x = (__bf16)lo;
    r.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// Two bf16 tensor additions' worth of one packed pair: bf16(a + b) per half,
// each a binary32 round-to-nearest add of exactly widened operands.
__device__ __forceinline__ uint32_t add_bf16x2(uint32_t a, uint32_t b)
{
    return pack_bf16(lo_f32(a) + lo_f32(b), hi_f32(a) + hi_f32(b));
}

__device__ __forceinline__ uint4 add_bf16x8(const uint4& a, const uint4& b)
{
    return make_uint4(add_bf16x2(a.x, b.x), add_bf16x2(a.y, b.y), add_bf16x2(a.z, b.z),
                      add_bf16x2(a.w, b.w));
}

// c + a.lo*b.lo + a.hi*b.hi on packed bf16 pairs (v_dot2_f32_bf16).  The
// bf16 products are exact in binary32; the sum is rounded by the instruction.
// Used for the per-source partial sums, whose accuracy need only be far below
// one bf16 ulp of the output.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                           c, false);
}

// ---- wave-wide sums -------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Maximum over each 16-lane DPP row, returned in all 16 lanes.  All 64 lanes
// must be active.
__device__ __forceinline__ float row_max(float v)
{
    v = fmaxf(v, dpp<0xb1>(v));
    v = fmaxf(v, dpp<0x4e>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return v;
}

// Maximum over the 64 lanes of a wave, in every lane (the four row maxima read
// as scalars).  All 64 lanes must be active.
__device__ __forceinline__ float wave_max(float v)
{
    v = row_max(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Wave totals of V per-lane values (V a power of two, <= 64) by a butterfly
// that halves each lane's list at every step: at step s lanes pair across
// lane bit 5 - s, the lane with that bit clear keeps the lower half of the
// list (its own plus its partner's) and the other lane the upper half, so
// after log2(V) steps lane v * (64 / V) holds the total of value v, and the
// remaining steps add the partner's copy.  The two steps across 16-lane rows
// use gfx950's v_permlane32_swap / v_permlane16_swap: given (lower half, upper
// half), the swap leaves in each lane the two terms of the half it keeps, so
// a pair costs one swap and one add.  The four steps within a row use DPP row
// permutations (row_mirror across bit 3, row_half_mirror across bit 2,
// quad_perm across bits 1 and 0; each partner has the same higher bits as its
// lane) and a select of the half to send.  Where both partners end with the
// same total they add the same two values, so it has the same bits in both.
// All 64 lanes must be active.
template <int STEP>
__device__ __forceinline__ float bfly_dpp(float v)
{
    if constexpr (STEP == 2)
        return dpp<0x140>(v); // row_mirror: lane i <-> 15 - i within a row
    else if constexpr (STEP == 3)
        return dpp<0x141>(v); // row_half_mirror: i <-> 7 - i within 8 lanes
    else if constexpr (STEP == 4)
        return dpp<0x4e>(v); // quad_perm [2,3,0,1]
    else
        return dpp<0xb1>(v); // quad_perm [1,0,3,2]
}

// Steps 0 and 1: lanes 0-31 keep lo and receive lo from lanes 32-63, which
// keep hi and receive hi from lanes 0-31 (step 0); the same between even and
// odd rows (step 1).  Returns the sum of the two terms each lane keeps.
template <int STEP>
__device__ __forceinline__ float bfly_swap_add(float lo, float hi)
{
    if constexpr (STEP == 0) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

template <int L, int STEP>
__device__ __forceinline__ void bfly_steps(float* w, int lane)
{
    if constexpr (STEP < 6) {
        if constexpr (L > 1) {
            if constexpr (STEP < 2) {
#pragma unroll
                for (int i = 0; i < L / 2; ++i)
                    w[i] = bfly_swap_add<STEP>(w[i], w[i + L / 2]);
            } else {
                const bool upper = (lane >> (5 - STEP)) & 1;
#pragma unroll
                for (int i = 0; i < L / 2; ++i) {
                    const float keep = upper ? w[i + L / 2] : w[i];
                    const float send = upper ? w[i] : w[i + L / 2];
                    w[i] = keep + bfly_dpp<STEP>(send);
                }
            }
            bfly_steps<L / 2, STEP + 1>(w, lane);
        } else {
            if constexpr (STEP < 2)
                w[0] = bfly_swap_add<STEP>(w[0], w[0]);
            else
                w[0] = w[0] + bfly_dpp<STEP>(w[0]);
            bfly_steps<1, STEP + 1>(w, lane);
        }
    }
}

constexpr int pow2_at_least(int n) { return n <= 1 ? 1 : 2 * pow2_at_least((n + 1) / 2); }

// The value whose total wave_totals leaves in `lane`, or -1 where the lane
// holds another lane's copy.
template <int V>
__device__ __forceinline__ int bfly_index(int lane)
{
    return lane % (64 / V) == 0 ? lane / (64 / V) : -1;
}

template <int NV>
__device__ __forceinline__ float wave_totals(const float (&part)[NV], int lane)
{
    constexpr int V = pow2_at_least(NV);
    static_assert(V <= 64, "one lane per value");
    float w[V];
#pragma unroll
    for (int i = 0; i < V; ++i)
        w[i] = i < NV ? part[i % NV] : 0.f;
    bfly_steps<V, 0>(w, lane);
    return w[0];
}

// Sum over the 64 lanes of a wave, returned identically (bit for bit) in every
// lane: the butterfly with one value, so every step adds the partner's copy
// (two lane swaps across rows, four DPP steps within them).  All 64 lanes must
// be active.
__device__ __forceinline__ float wave_sum(float v)
{
    const float part[1] = {v};
    return wave_totals<1>(part, 0);
}

// ---- cross-workgroup exchange --------------------------------------------
//
// Workgroups that share a token exchange binary32 partial sums through 64-bit
// records: the upper word is a tag, the lower word the value.  A record is
// written with single 8-byte atomic stores and read with relaxed device-scope
// atomic loads, so a reader that sees the expected tag also sees that call's
// value: no fence (and none of the whole-cache writeback/invalidate that
// device-scope release/acquire costs on gfx950) is needed.  Tags come from a
// per-token epoch word that advances once per call (see fwd_split), so records
// left by earlier calls never match: tag 0 (a record never written) is never
// expected, and the call that wraps the epoch clears the records of every
// chunk index it does not use (see advance_epoch).
//
// Every record is written twice.  The first copy, at `rec`, takes a
// workgroup-scope store: it goes no further than the L2 of the writer's XCD,
// where the device-scope loads of the other CUs of that XCD see it (one hop
// of about 190 ns on an idle device against 292 for a device-scope store, and
// it does not queue behind the whole chip's memory traffic when the other CUs
// stream).  The second, at rec + dev_off, takes a device-scope store and is
// seen from every XCD.  Readers poll the first copy for a bounded number of
// re-polls, then the second (see fwd_split): the chunks of a token are placed
// on one XCD, so the first copy is the one that arrives, but the result never
// depends on where the workgroups run, since a record with the expected tag
// is taken from either copy and both hold the same bits.

__device__ __forceinline__ void publish(unsigned long long* rec, int dev_off, unsigned tag, float v)
{
    const unsigned long long w = ((unsigned long long)tag << 32) | __float_as_uint(v);
    __hip_atomic_store(rec, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_store(rec + dev_off, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned long long peek(const unsigned long long* rec)
{
    return __hip_atomic_load(const_cast<unsigned long long*>(rec), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ unsigned tag_of(unsigned long long w) { return (unsigned)(w >> 32); }

} // namespace attnres
