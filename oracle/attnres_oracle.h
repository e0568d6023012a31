/*
 * CPU oracle for the fused attention-residual (AttnRes) combine + RMSNorm with
 * the MoE-tail additions folded in.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load or call this library; the product
 * path (the HIP library and its Python binding) never does.  It shares no code
 * with the HIP path: no headers, helpers, tables or constants.
 *
 * All tensors are host arrays of bf16 bit patterns (uint16_t), row-major
 * [M, H] unless stated otherwise.  Floating-point work is binary64 except the
 * prefix fold-add, which the source fixes to binary32 round-to-nearest adds.
 *
 * Parity pins: every function below is pinned by the CPU tests (exhaustive
 * rounding checks, library comparisons, closed forms and invariants).  The
 * mixing formula itself is not printed by the source pages; its fidelity to
 * the real model layer is "parity unpinned" (see the header of the .c file).
 */
#ifndef ATTNRES_ORACLE_H
#define ATTNRES_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Round a binary64 value to the nearest bf16 (ties to even), with gradual
 * underflow and overflow to +-Inf.  NaN maps to a quiet NaN with its sign. */
uint16_t oracle_round_bf16(double x);

/* Exact widening of a bf16 bit pattern to binary64. */
double oracle_bf16_to_f64(uint16_t b);

/* One bf16 tensor addition element: bf16(f32(a) + f32(b)), the binary32 add
 * rounding to nearest even with subnormals kept. */
uint16_t oracle_bf16_add(uint16_t a, uint16_t b);

/* Elementwise bf16 tensor addition out[i] = oracle_bf16_add(a[i], b[i]). */
void oracle_bf16_add_tensor(const uint16_t* a, const uint16_t* b, uint16_t* out,
                            int64_t n);

/* The whole fused operation for M tokens.
 *   prefix, add      [M,H]  required
 *   add2             [M,H]  or NULL (no second addend)
 *   snapshots        host array of n_snapshots pointers, each [M,H]
 *   query, gamma     [H]
 *   out_prefix       [M,H]  updated prefix, bit-exact definition
 *   out_norm         [M,H]  RMSNorm'd mixture rounded once to bf16
 *   out_norm_f64     [M,H]  or NULL: the same before the final rounding
 *   alpha            [M, n_snapshots+1] or NULL: softmax weights, source order
 *                    snapshots 0..N-1 then the updated prefix
 * Returns 0, or -1 on a bad argument (null pointer, M<0, H<=0, N<0). */
int oracle_attnres_fwd(const uint16_t* prefix, const uint16_t* add,
                       const uint16_t* add2, const uint16_t* const* snapshots,
                       int n_snapshots, const uint16_t* query,
                       const uint16_t* gamma, float eps, int64_t M, int64_t H,
                       uint16_t* out_prefix, uint16_t* out_norm,
                       double* out_norm_f64, double* alpha);

/* The same operation with the pre-norm mixture as well (the speculative-decoding
 * capture tap of the source page's "Model" section needs it):
 *   out_mix          [M,H]  or NULL: x = sum_s alpha_s k_s rounded once to bf16
 *   out_mix_f64      [M,H]  or NULL: x before the rounding
 * Every other argument and the return value as oracle_attnres_fwd. */
int oracle_attnres_fwd_mix(const uint16_t* prefix, const uint16_t* add,
                           const uint16_t* add2, const uint16_t* const* snapshots,
                           int n_snapshots, const uint16_t* query,
                           const uint16_t* gamma, float eps, int64_t M, int64_t H,
                           uint16_t* out_prefix, uint16_t* out_norm, uint16_t* out_mix,
                           double* out_norm_f64, double* out_mix_f64, double* alpha);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_ORACLE_H */
