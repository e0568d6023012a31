// Device self-test of the rounding the kernels rely on: gfx950's packed
// binary32 -> bf16 conversion (pack_bf16) against rounding by definition on the
// bit pattern, over every binary32 input.  The kernels' results are bit-exact
// only if the two agree (the fold-add of page "[#20545][perf] Kimi K3: fold the
// MoE-tail additions into the next attention-residual", section "Op", asks for
// round-to-nearest additions with subnormals kept).
#include "attnres.h"
#include "attnres_device.hpp"

#include <hip/hip_runtime.h>

namespace attnres {

// Rounding by definition: keep the upper 16 bits, step up when the dropped
// half is above one half, or equal to it with an odd kept half.
__device__ __forceinline__ uint32_t round_by_definition(uint32_t u)
{
    uint32_t keep = u >> 16;
    const uint32_t drop = u & 0xffffu;
    if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u)))
        keep += 1u;
    return keep;
}

__device__ __forceinline__ bool is_nan16(uint32_t h) { return ((h & 0x7f80u) == 0x7f80u) && (h & 0x7fu); }

// Thread i checks inputs 2i, 2i+1, 2i + 2n, ... (n = total threads): every
// 32-bit pattern exactly once.  Mismatch counts go to counts[0] (non-NaN
// inputs) and counts[1] (NaN inputs that did not give a NaN).
__global__ __launch_bounds__(256) void selftest_rounding_kernel(unsigned long long* counts)
{
    const uint64_t n = (uint64_t)gridDim.x * blockDim.x;
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    unsigned long long bad = 0, badnan = 0;
    for (uint64_t i = 2 * tid; i < (uint64_t(1) << 32); i += 2 * n) {
        const uint32_t u0 = (uint32_t)i, u1 = (uint32_t)(i + 1);
        const uint32_t w = pack_bf16(__uint_as_float(u0), __uint_as_float(u1));
        const uint32_t h[2] = {w & 0xffffu, w >> 16};
        const uint32_t u[2] = {u0, u1};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            if ((u[e] & 0x7fffffffu) > 0x7f800000u)
                badnan += is_nan16(h[e]) ? 0 : 1;
            else
                bad += h[e] == round_by_definition(u[e]) ? 0 : 1;
        }
    }
    if (bad)
        atomicAdd(&counts[0], bad);
    if (badnan)
        atomicAdd(&counts[1], badnan);
}

} // namespace attnres

extern "C" int attnres_selftest_rounding(unsigned long long* mismatches)
{
    if (!mismatches)
        return ATTNRES_EINVAL;
    unsigned long long* d = nullptr;
    if (hipMalloc(&d, 2 * sizeof(unsigned long long)) != hipSuccess)
        return ATTNRES_EHIP;
    int rc = ATTNRES_OK;
    unsigned long long h[2] = {0, 0};
    if (hipMemset(d, 0, sizeof h) != hipSuccess)
        rc = ATTNRES_EHIP;
    if (rc == ATTNRES_OK) {
        hipLaunchKernelGGL(attnres::selftest_rounding_kernel, dim3(4096), dim3(256), 0, 0, d);
        if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
            hipMemcpy(h, d, sizeof h, hipMemcpyDeviceToHost) != hipSuccess)
            rc = ATTNRES_EHIP;
    }
    (void)hipFree(d);
    *mismatches = h[0] + h[1];
    return rc;
}
