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
//   W  one workgroup per token: the token's whole row set is held in
//      registers (N+1 sources x 8 bf16 x VPT 16-byte vectors per thread), the
//      2(N+1) partials are reduced wave-wide on DPP and across waves in LDS.
//      No inter-workgroup communication.  Used when there are many tokens.
//   S  split hidden: C single-wave workgroups per token, each owning 64*VPT
//      16-byte vectors of the row.  Partials go through a device scratch
//      buffer and a per-token barrier (two per call: after A2 and after the
//      sum of squares of A5).  Spreads a few tokens over many CUs, which is
//      what the latency-bound small-M calls need.
// Both reduce in a fixed order: the same inputs give the same bits, and the
// add2 / no-add2 instantiations share every line after A1.
#include "attnres.h"
#include "attnres_device.hpp"
#include "attnres_host.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <utility>

namespace attnres {

constexpr int PART_STRIDE = 32;          // floats per (token, chunk) partial record (>= 2*13)
constexpr int SYNC_STRIDE = 32;          // barrier words per token: one 128-byte line each
constexpr unsigned SPIN_LIMIT = 1u << 20;

struct Params {
    const uint4* prefix;
    const uint4* add;
    const uint4* add2;
    const uint4* snap[MAX_SNAP];
    const uint4* query;
    const uint4* gamma;
    uint4* out_prefix;
    uint4* out_norm;
    float eps;
    float inv_h;        // 1/H: mean = sum * inv_h
    int nvec;           // H / 8 (16-byte vectors per row)
    int chunks;         // split hidden: workgroups per token
    int64_t M;
    float* part;        // split hidden: [token][chunk][PART_STRIDE] partials of A2
    float* part2;       // split hidden: [token][chunk] sum of squares of the mixture
    unsigned* sync;     // split hidden: [token][SYNC_STRIDE] barrier words
    unsigned* timeouts; // split hidden: barrier polls that gave up
    unsigned spin_limit;
};

// Softmax weights from the reduced partials tot[2s] = sum k^2, tot[2s+1] = q.k.
template <int S>
__device__ __forceinline__ void softmax_weights(const float* tot, float inv_h, float eps, float* alpha)
{
    float z[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const float rstd = rsqrtf(tot[2 * s] * inv_h + eps);
        z[s] = rstd * tot[2 * s + 1];
    }
    float zmax = z[0];
#pragma unroll
    for (int s = 1; s < S; ++s)
        zmax = fmaxf(zmax, z[s]);
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
        alpha[s] = __expf(z[s] - zmax);
        sum += alpha[s];
    }
    const float inv = 1.0f / sum;
#pragma unroll
    for (int s = 0; s < S; ++s)
        alpha[s] = alpha[s] * inv;
}

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
    a = p.prefix[row + vc];
    b = p.add[row + vc];
    c = ADD2 ? p.add2[row + vc] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int s = 0; s < NS; ++s)
        k[s][j] = p.snap[s][row + vc];
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

// A2 for one thread: per-source sums over its VPT*8 elements in a fixed order
// (vector by vector, pair by pair, on v_dot2_f32_bf16); vectors outside the
// row (ok[j] false) contribute zero.
template <int S, int VPT>
__device__ __forceinline__ void source_partials(const uint4 (&k)[S][VPT], const uint4* q, const bool* ok,
                                                float* part)
{
#pragma unroll
    for (int s = 0; s < S; ++s) {
        float ss = 0.f, qd = 0.f;
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const uint4 x = k[s][j];
            float ssj = dot2_bf16(x.x, x.x, 0.f);
            ssj = dot2_bf16(x.y, x.y, ssj);
            ssj = dot2_bf16(x.z, x.z, ssj);
            ssj = dot2_bf16(x.w, x.w, ssj);
            float qdj = dot2_bf16(q[j].x, x.x, 0.f);
            qdj = dot2_bf16(q[j].y, x.y, qdj);
            qdj = dot2_bf16(q[j].z, x.z, qdj);
            qdj = dot2_bf16(q[j].w, x.w, qdj);
            ss += ok[j] ? ssj : 0.f;
            qd += ok[j] ? qdj : 0.f;
        }
        part[2 * s] = ss;
        part[2 * s + 1] = qd;
    }
}

// Workgroup-wide sums of NV per-thread values; afterwards tot[0..NV-1] (LDS)
// holds the totals, which every thread reads with identical bits.  Quads are
// summed first (DPP); one lane per quad stores its NV quad sums as a row of
// `rows` (NVP floats, zero padded); fixed segments of rows are summed by
// (value, segment) threads, and the segment sums in segment order.  The order
// is fixed by (NV, blockDim.x) alone.
template <int NV, int NVP>
__device__ __forceinline__ void block_sums(float (&part)[NV], float* rows, float* segs, float* tot, int tid,
                                           int nthreads)
{
#pragma unroll
    for (int i = 0; i < NV; ++i)
        part[i] = quad_sum(part[i]);
    if ((tid & 3) == 0) {
        float4* r = reinterpret_cast<float4*>(rows + (tid >> 2) * NVP);
#pragma unroll
        for (int i = 0; i < NVP / 4; ++i)
            r[i] = make_float4(4 * i + 0 < NV ? part[(4 * i + 0) % NV] : 0.f,
                               4 * i + 1 < NV ? part[(4 * i + 1) % NV] : 0.f,
                               4 * i + 2 < NV ? part[(4 * i + 2) % NV] : 0.f,
                               4 * i + 3 < NV ? part[(4 * i + 3) % NV] : 0.f);
    }
    __syncthreads();
    const int nrows = nthreads >> 2;
    const int nseg = nthreads / NVP;
    const int rps = (nrows + nseg - 1) / nseg;
    if (tid < nseg * NVP) {
        const int v = tid % NVP, seg = tid / NVP;
        const int r0 = seg * rps, r1 = min(nrows, r0 + rps);
        float acc = 0.f;
        for (int r = r0; r < r1; ++r)
            acc += rows[r * NVP + v];
        segs[seg * NVP + v] = acc;
    }
    __syncthreads();
    if (tid < NV) {
        float acc = segs[tid];
        for (int sg = 1; sg < nseg; ++sg)
            acc += segs[sg * NVP + tid];
        tot[tid] = acc;
    }
    __syncthreads();
}

// A4 for one thread: x = sum_s alpha_s k_s (fixed source order), and the
// thread's share of sum x^2 (vectors outside the row contribute zero).
template <int S, int VPT>
__device__ __forceinline__ float combine(const uint4 (&k)[S][VPT], const float* alpha, const bool* ok,
                                         float (&x)[VPT][8])
{
    float sx = 0.f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        float sxj = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = alpha[0] * elem(k[0][j], e);
#pragma unroll
            for (int s = 1; s < S; ++s)
                acc = __builtin_fmaf(alpha[s], elem(k[s][j], e), acc);
            x[j][e] = acc;
            sxj = __builtin_fmaf(acc, acc, sxj);
        }
        sx += ok[j] ? sxj : 0.f;
    }
    return sx;
}

// A5 output of one vector: bf16((x * rstd) * gamma).
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
template <int NS, bool ADD2, int VPT, int MAXB>
__global__ __launch_bounds__(MAXB) void fwd_wg(Params p)
{
    constexpr int S = NS + 1;                // sources: snapshots, then the updated prefix
    constexpr int NV = 2 * S;                // partials per token
    constexpr int NVP = (NV + 3) / 4 * 4;    // LDS record length
    constexpr int MAXW = MAXB / 64;
    __shared__ __align__(16) float rows[(MAXB / 4) * NVP];
    __shared__ float segs[MAXB];
    __shared__ __align__(16) float tot[NVP];
    __shared__ float red2[MAXW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nthreads = blockDim.x;
    const int nw = nthreads >> 6;
    const int nvec = p.nvec;

    for (int64_t t = blockIdx.x; t < p.M; t += gridDim.x) {
        const int64_t row = t * (int64_t)nvec;
        uint4 k[S][VPT], q[VPT], g[VPT], a[VPT], b[VPT], c[VPT];
        bool ok[VPT];
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int v = tid + j * nthreads;
            ok[j] = v < nvec;
            load_vectors<NS, ADD2>(p, row, v, ok[j], a[j], b[j], c[j], k, j, q[j], g[j]);
        }
        // keep every load above this point: nothing that waits on a load may be
        // scheduled between them
        __builtin_amdgcn_sched_barrier(0);

        // A1
        fold_add<ADD2, VPT>(a, b, c, k[NS]);
#pragma unroll
        for (int j = 0; j < VPT; ++j)
            if (ok[j])
                p.out_prefix[row + tid + j * nthreads] = k[NS][j];

        // A2: per thread, then over the workgroup
        float part[NV];
        source_partials<S, VPT>(k, q, ok, part);
        fence_sources<S, VPT>(k);
        block_sums<NV, NVP>(part, rows, segs, tot, tid, nthreads);

        // A3
        float totr[NV], alpha[S];
#pragma unroll
        for (int i = 0; i < NV; ++i)
            totr[i] = tot[i];
        softmax_weights<S>(totr, p.inv_h, p.eps, alpha);

        // A4 + A5
        float x[VPT][8];
        const float sx = wave_sum(combine<S, VPT>(k, alpha, ok, x));
        if (lane == 0)
            red2[wave] = sx;
        __syncthreads();
        float ssum = red2[0];
        for (int w = 1; w < nw; ++w)
            ssum += red2[w];
        const float rstd = rsqrtf(ssum * p.inv_h + p.eps);
#pragma unroll
        for (int j = 0; j < VPT; ++j)
            if (ok[j])
                p.out_norm[row + tid + j * nthreads] = normalise(x[j], rstd, g[j]);
        __syncthreads(); // LDS reuse by the next token
    }
}

// ---------------------------------------------------------------------------
// Kernel S: split hidden.  Workgroup b (one wave) handles token b / C, chunk
// b % C, i.e. vectors chunk*64*VPT + j*64 + lane.  grid = M * C exactly.
template <int NS, bool ADD2, int VPT>
__global__ __launch_bounds__(64) void fwd_split(Params p)
{
    constexpr int S = NS + 1;
    constexpr int NV = 2 * S;
    constexpr int CV = 64 * VPT;

    const int lane = threadIdx.x;
    const int C = p.chunks;
    const int64_t t = blockIdx.x / C;
    const int chunk = (int)(blockIdx.x - t * C);
    const int nvec = p.nvec;
    const int64_t row = t * (int64_t)nvec;

    uint4 k[S][VPT], q[VPT], g[VPT], a[VPT], b[VPT], c[VPT];
    bool ok[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int v = chunk * CV + j * 64 + lane;
        ok[j] = v < nvec;
        load_vectors<NS, ADD2>(p, row, v, ok[j], a[j], b[j], c[j], k, j, q[j], g[j]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // A1
    fold_add<ADD2, VPT>(a, b, c, k[NS]);
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        if (ok[j])
            p.out_prefix[row + chunk * CV + j * 64 + lane] = k[NS][j];

    // A2: thread -> wave; lane i publishes partial i of this chunk
    float part[NV];
    source_partials<S, VPT>(k, q, ok, part);
    fence_sources<S, VPT>(k);
    float mine = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const float w = wave_sum(part[i]);
        mine = (lane == i) ? w : mine;
    }
    float* rec = p.part + (size_t)t * C * PART_STRIDE;
    if (lane < NV)
        store_agent(&rec[chunk * PART_STRIDE + lane], mine);
    unsigned* sync = p.sync + (size_t)t * SYNC_STRIDE;
    token_barrier(sync, (unsigned)C, p.spin_limit, p.timeouts);

    // every workgroup of the token sums the chunk records in chunk order
    float acc = 0.f;
    if (lane < NV) {
        acc = load_agent(&rec[lane]);
        for (int cc = 1; cc < C; ++cc)
            acc += load_agent(&rec[cc * PART_STRIDE + lane]);
    }
    float tot[NV], alpha[S];
#pragma unroll
    for (int i = 0; i < NV; ++i)
        tot[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), i));

    // A3, A4
    softmax_weights<S>(tot, p.inv_h, p.eps, alpha);
    float x[VPT][8];
    const float sx = wave_sum(combine<S, VPT>(k, alpha, ok, x));
    if (lane == 0)
        store_agent(&p.part2[(size_t)t * C + chunk], sx);
    token_barrier(sync, (unsigned)C, p.spin_limit, p.timeouts);

    // A5
    const float h = lane < C ? load_agent(&p.part2[(size_t)t * C + lane]) : 0.f;
    const float ssum = wave_sum(h);
    const float rstd = rsqrtf(ssum * p.inv_h + p.eps);
#pragma unroll
    for (int j = 0; j < VPT; ++j)
        if (ok[j])
            p.out_norm[row + chunk * CV + j * 64 + lane] = normalise(x[j], rstd, g[j]);
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

template <bool A2, int VPT, int MAXB, int... I>
constexpr std::array<Kernel, sizeof...(I)> wg_table(std::integer_sequence<int, I...>)
{
    return {{&fwd_wg<I, A2, VPT, MAXB>...}};
}

template <bool A2, int VPT, int... I>
constexpr std::array<Kernel, sizeof...(I)> split_table(std::integer_sequence<int, I...>)
{
    return {{&fwd_split<I, A2, VPT>...}};
}

using Seq = std::make_integer_sequence<int, MAX_SNAP + 1>;

// [add2][N]
const std::array<Kernel, MAX_SNAP + 1> kWg1[2] = {wg_table<false, 1, 1024>(Seq{}), wg_table<true, 1, 1024>(Seq{})};
const std::array<Kernel, MAX_SNAP + 1> kWg2[2] = {wg_table<false, 2, 512>(Seq{}), wg_table<true, 2, 512>(Seq{})};
const std::array<Kernel, MAX_SNAP + 1> kWg4[2] = {wg_table<false, 4, 512>(Seq{}), wg_table<true, 4, 512>(Seq{})};
const std::array<Kernel, MAX_SNAP + 1> kSp1[2] = {split_table<false, 1>(Seq{}), split_table<true, 1>(Seq{})};
const std::array<Kernel, MAX_SNAP + 1> kSp2[2] = {split_table<false, 2>(Seq{}), split_table<true, 2>(Seq{})};

struct Scratch {
    void* base = nullptr;
    float* part = nullptr;
    float* part2 = nullptr;
    unsigned* sync = nullptr;
    unsigned* timeouts = nullptr;
};

constexpr int MAX_DEVICES = 64;
std::mutex g_mutex;
Scratch g_scratch[MAX_DEVICES];
int g_force_variant = 0;
int g_force_param = 0;

constexpr size_t PART_BYTES = sizeof(float) * MAX_SPLIT_TOKENS * MAX_CHUNKS * PART_STRIDE;
constexpr size_t PART2_BYTES = sizeof(float) * MAX_SPLIT_TOKENS * MAX_CHUNKS;
constexpr size_t SYNC_BYTES = sizeof(unsigned) * MAX_SPLIT_TOKENS * SYNC_STRIDE;
constexpr size_t SCRATCH_BYTES = PART_BYTES + PART2_BYTES + SYNC_BYTES + 256;

// The scratch of the current device, allocated and cleared on first use.
int scratch_for_current_device(Scratch** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
        return ATTNRES_EHIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    Scratch& s = g_scratch[dev];
    if (!s.base) {
        void* base = nullptr;
        if (hipMalloc(&base, SCRATCH_BYTES) != hipSuccess)
            return ATTNRES_EHIP;
        if (hipMemset(base, 0, SCRATCH_BYTES) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
            (void)hipFree(base);
            return ATTNRES_EHIP;
        }
        char* c = static_cast<char*>(base);
        s.part = reinterpret_cast<float*>(c);
        s.part2 = reinterpret_cast<float*>(c + PART_BYTES);
        s.sync = reinterpret_cast<unsigned*>(c + PART_BYTES + PART2_BYTES);
        s.timeouts = reinterpret_cast<unsigned*>(c + PART_BYTES + PART2_BYTES + SYNC_BYTES);
        s.base = base;
    }
    *out = &s;
    return ATTNRES_OK;
}

} // namespace attnres

using namespace attnres;

extern "C" int attnres_add_rmsnorm_fwd(const void* prefix, const void* add, const void* add2,
                                       const void* const* snapshots, int n_snapshots,
                                       const void* query, const void* gamma, float eps, int64_t M,
                                       int64_t H, void* out_prefix, void* out_norm,
                                       hipStream_t stream)
{
    int rc = validate_fwd(prefix, add, add2, snapshots, n_snapshots, query, gamma, eps, M, H,
                          out_prefix, out_norm);
    if (rc != ATTNRES_OK)
        return rc;
    Plan pl;
    rc = make_plan(M, n_snapshots, H, g_force_variant, g_force_param, pl);
    if (rc != ATTNRES_OK)
        return rc;
    if (M == 0)
        return ATTNRES_OK;

    Params p{};
    p.prefix = static_cast<const uint4*>(prefix);
    p.add = static_cast<const uint4*>(add);
    p.add2 = static_cast<const uint4*>(add2);
    for (int s = 0; s < n_snapshots; ++s)
        p.snap[s] = static_cast<const uint4*>(snapshots[s]);
    p.query = static_cast<const uint4*>(query);
    p.gamma = static_cast<const uint4*>(gamma);
    p.out_prefix = static_cast<uint4*>(out_prefix);
    p.out_norm = static_cast<uint4*>(out_norm);
    p.eps = eps;
    p.inv_h = 1.0f / (float)H;
    p.nvec = (int)(H / 8);
    p.chunks = pl.chunks;
    p.M = M;
    p.spin_limit = SPIN_LIMIT;

    const int a2 = add2 ? 1 : 0;
    Kernel fn = nullptr;
    if (pl.variant == 2) {
        Scratch* sc = nullptr;
        rc = scratch_for_current_device(&sc);
        if (rc != ATTNRES_OK)
            return rc;
        p.part = sc->part;
        p.part2 = sc->part2;
        p.sync = sc->sync;
        p.timeouts = sc->timeouts;
        fn = (pl.vpt == 1 ? kSp1 : kSp2)[a2][n_snapshots];
    } else {
        fn = (pl.vpt == 1 ? kWg1 : pl.vpt == 2 ? kWg2 : kWg4)[a2][n_snapshots];
    }
    void* args[] = {&p};
    if (hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3((unsigned)pl.grid), dim3(pl.threads),
                        args, 0, stream) != hipSuccess)
        return ATTNRES_EHIP;
    return ATTNRES_OK;
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
    Scratch* sc = nullptr;
    return scratch_for_current_device(&sc);
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

extern "C" const char* attnres_status_string(int status)
{
    switch (status) {
    case ATTNRES_OK: return "ok";
    case ATTNRES_EINVAL: return "invalid argument";
    case ATTNRES_EUNSUPPORTED: return "unsupported (more than 12 snapshots): add first, use the unfused route";
    case ATTNRES_EALIAS: return "forbidden buffer overlap";
    case ATTNRES_EHIP: return "HIP error";
    default: return "unknown status";
    }
}

extern "C" int attnres_version(void) { return 100; }
