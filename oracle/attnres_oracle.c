/*
 * CPU oracle: fused attention-residual (AttnRes) combine + RMSNorm with the
 * MoE-tail additions folded in.  Plain, slow, obviously correct.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the
 * benchmark).  Shares no code with the HIP path.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off (no FTZ/DAZ start-up code,
 * binary32 arithmetic evaluated in binary32 on x86-64 SSE).
 *
 * What it computes, per token m (rows are independent):
 *
 *  1. Fold-add.  Page "[#20545][perf] Kimi K3: fold the MoE-tail additions
 *     into the next attention-residual" (TensorRT-LLM #20546), sections
 *     "Description" and "Op": a MoE layer ends with prefix + (routed + shared);
 *     the fused op takes the two addends and produces the updated prefix as
 *     bf16(prefix + bf16(add + add2)), each addition a binary32
 *     round-to-nearest add, subnormals kept, identical bit for bit to two bf16
 *     tensor additions.  Without add2 the update is bf16(prefix + add).
 *
 *  2. Mix.  The same page names the consumer an "attention-residual" and,
 *     in section "Model", says the hidden-state capture needs the pre-norm
 *     mixture, but prints no formula.  Reading adopted here (parity with the
 *     real model layer is "parity unpinned"): the sources are the N snapshot
 *     rows followed by the bf16-rounded updated prefix; each source k_s gets
 *     the logit z_s = q . (k_s / sqrt(mean(k_s^2) + eps)) with a weightless
 *     key RMSNorm and no temperature; alpha = softmax(z) over the N+1
 *     sources; the mixture is x = sum_s alpha_s k_s over the raw sources.
 *
 *  3. Final RMSNorm.  Named by the same page ("attention-residual +
 *     RMSNorm"); the plain form y = x / sqrt(mean(x^2) + eps) * gamma, gamma
 *     used as the full weight, rounded once to bf16.
 *
 * Steps 2 and 3 run in binary64 with one rounding at the end.
 */
#include "attnres_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static float bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Nearest bf16 by definition: find the binade of |x|, take the bf16 quantum
 * there (2^(E-7) for normal binades, 2^-133 for the subnormal range), divide
 * (exact: a power-of-two scaling), round the quotient to the nearest integer
 * with ties to even (nearbyint under the default rounding mode), multiply
 * back.  The result is a bf16 value, hence exactly representable in binary32.
 */
uint16_t oracle_round_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;

    int e;
    frexp(a, &e);        /* a in [2^(e-1), 2^e) */
    int E = e - 1;       /* a in [2^E, 2^(E+1)) */
    if (E < -126)
        E = -126;        /* subnormal bf16 values share the quantum 2^-133 */
    double quantum = ldexp(1.0, E - 7);
    double n = nearbyint(a / quantum);
    double y = n * quantum;
    if (y >= 0x1p128)
        return (uint16_t)(sign | 0x7F80u);
    if (y == 0.0)
        return sign;

    float f = (float)y; /* exact: y is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

uint16_t oracle_bf16_add(uint16_t a, uint16_t b)
{
    volatile float s = bf16_to_f32(a) + bf16_to_f32(b); /* binary32 RN add */
    return oracle_round_bf16((double)s);
}

void oracle_bf16_add_tensor(const uint16_t* a, const uint16_t* b, uint16_t* out,
                            int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_add(a[i], b[i]);
}

/* One token.  k: scratch of (N+2)*H doubles (the sources, then the mixture). */
static void one_token(const uint16_t* prefix, const uint16_t* add,
                      const uint16_t* add2, const uint16_t* const* snap_rows,
                      int N, const uint16_t* query, const uint16_t* gamma,
                      double eps, int64_t H, uint16_t* out_prefix,
                      uint16_t* out_norm, uint16_t* out_mix, double* out_norm_f64,
                      double* out_mix_f64, double* alpha, double* k, double* z)
{
    /* 1. fold-add: the updated prefix, bit-exact */
    for (int64_t h = 0; h < H; ++h) {
        uint16_t t = add2 ? oracle_bf16_add(add[h], add2[h]) : add[h];
        out_prefix[h] = oracle_bf16_add(prefix[h], t);
    }

    /* sources, widened exactly: snapshots 0..N-1, then the rounded prefix */
    int S = N + 1;
    for (int s = 0; s < N; ++s)
        for (int64_t h = 0; h < H; ++h)
            k[(int64_t)s * H + h] = oracle_bf16_to_f64(snap_rows[s][h]);
    for (int64_t h = 0; h < H; ++h)
        k[(int64_t)N * H + h] = oracle_bf16_to_f64(out_prefix[h]);

    /* 2. logits: query . RMSNorm(source) */
    for (int s = 0; s < S; ++s) {
        const double* ks = k + (int64_t)s * H;
        double sumsq = 0.0, qdot = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            sumsq += ks[h] * ks[h];
            qdot += oracle_bf16_to_f64(query[h]) * ks[h];
        }
        double rstd = 1.0 / sqrt(sumsq / (double)H + eps);
        z[s] = rstd * qdot;
    }

    /* softmax over the sources, with the maximum subtracted */
    double zmax = z[0];
    for (int s = 1; s < S; ++s)
        if (z[s] > zmax)
            zmax = z[s];
    double denom = 0.0;
    for (int s = 0; s < S; ++s) {
        z[s] = exp(z[s] - zmax);
        denom += z[s];
    }
    for (int s = 0; s < S; ++s) {
        z[s] = z[s] / denom;
        if (alpha)
            alpha[s] = z[s];
    }

    /* weighted combine of the raw sources, then the final RMSNorm */
    double sumsq = 0.0;
    for (int64_t h = 0; h < H; ++h) {
        double x = 0.0;
        for (int s = 0; s < S; ++s)
            x += z[s] * k[(int64_t)s * H + h];
        k[(int64_t)S * H + h] = x; /* one spare row holds the mixture */
        if (out_mix_f64)
            out_mix_f64[h] = x;
        if (out_mix)
            out_mix[h] = oracle_round_bf16(x); /* the pre-norm mixture, rounded once */
        sumsq += x * x;
    }
    double rstd = 1.0 / sqrt(sumsq / (double)H + eps);
    for (int64_t h = 0; h < H; ++h) {
        double y = k[(int64_t)S * H + h] * rstd * oracle_bf16_to_f64(gamma[h]);
        if (out_norm_f64)
            out_norm_f64[h] = y;
        out_norm[h] = oracle_round_bf16(y);
    }
}

int oracle_attnres_fwd(const uint16_t* prefix, const uint16_t* add,
                       const uint16_t* add2, const uint16_t* const* snapshots,
                       int n_snapshots, const uint16_t* query,
                       const uint16_t* gamma, float eps, int64_t M, int64_t H,
                       uint16_t* out_prefix, uint16_t* out_norm,
                       double* out_norm_f64, double* alpha)
{
    return oracle_attnres_fwd_mix(prefix, add, add2, snapshots, n_snapshots, query,
                                  gamma, eps, M, H, out_prefix, out_norm, NULL,
                                  out_norm_f64, NULL, alpha);
}

int oracle_attnres_fwd_mix(const uint16_t* prefix, const uint16_t* add,
                           const uint16_t* add2, const uint16_t* const* snapshots,
                           int n_snapshots, const uint16_t* query,
                           const uint16_t* gamma, float eps, int64_t M, int64_t H,
                           uint16_t* out_prefix, uint16_t* out_norm, uint16_t* out_mix,
                           double* out_norm_f64, double* out_mix_f64, double* alpha)
{
    if (!prefix || !add || !query || !gamma || !out_prefix || !out_norm)
        return -1;
    if (M < 0 || H <= 0 || n_snapshots < 0)
        return -1;
    if (n_snapshots > 0 && !snapshots)
        return -1;
    for (int s = 0; s < n_snapshots; ++s)
        if (!snapshots[s])
            return -1;
    if (M == 0)
        return 0;

    int S = n_snapshots + 1;
    double* k = (double*)malloc(sizeof(double) * (size_t)(S + 1) * (size_t)H);
    double* z = (double*)malloc(sizeof(double) * (size_t)S);
    const uint16_t** rows =
        (const uint16_t**)malloc(sizeof(uint16_t*) * (size_t)(n_snapshots + 1));
    if (!k || !z || !rows) {
        free(k);
        free(z);
        free(rows);
        return -2;
    }
    double eps_d = (double)eps;

    for (int64_t m = 0; m < M; ++m) {
        int64_t off = m * H;
        for (int s = 0; s < n_snapshots; ++s)
            rows[s] = snapshots[s] + off;
        one_token(prefix + off, add + off, add2 ? add2 + off : NULL, rows,
                  n_snapshots, query, gamma, eps_d, H, out_prefix + off,
                  out_norm + off, out_mix ? out_mix + off : NULL,
                  out_norm_f64 ? out_norm_f64 + off : NULL,
                  out_mix_f64 ? out_mix_f64 + off : NULL,
                  alpha ? alpha + m * S : NULL, k, z);
    }
    free(k);
    free(z);
    free(rows);
    return 0;
}
