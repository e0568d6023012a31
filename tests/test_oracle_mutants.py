"""CPU mutation check of the oracle's pins.

Each mutant plants one plausible mistake in a copy of the oracle source (a
dropped rounding, a flushed subnormal, a missing key RMSNorm, a flipped sign,
a wrong row ...), builds it into a temporary library and runs the pins: at
least one pin must fail.  This shows the pins would catch that mistake in the
oracle.  Mistakes are planted only here, on the CPU.
"""
import os

import pytest

import oracle
import pins
from oracle import build as obuild

SRC = open(obuild.SOURCE).read()

# name -> (exact text in the oracle source, replacement)
MUTANTS = {
    "inner_rounding_dropped": (
        "        uint16_t t = add2 ? oracle_bf16_add(add[h], add2[h]) : add[h];\n"
        "        out_prefix[h] = oracle_bf16_add(prefix[h], t);",
        "        volatile float s3 = bf16_to_f32(prefix[h]) + (bf16_to_f32(add[h]) +\n"
        "                            (add2 ? bf16_to_f32(add2[h]) : 0.0f));\n"
        "        out_prefix[h] = oracle_round_bf16((double)s3);"),
    "addends_reassociated": (
        "        uint16_t t = add2 ? oracle_bf16_add(add[h], add2[h]) : add[h];\n"
        "        out_prefix[h] = oracle_bf16_add(prefix[h], t);",
        "        uint16_t t = oracle_bf16_add(prefix[h], add[h]);\n"
        "        out_prefix[h] = add2 ? oracle_bf16_add(t, add2[h]) : t;"),
    "flush_to_zero": (
        "    volatile float s = bf16_to_f32(a) + bf16_to_f32(b); /* binary32 RN add */",
        "    volatile float s = bf16_to_f32(a) + bf16_to_f32(b);\n"
        "    if (fabsf(s) < 0x1p-126f) s = 0.0f;"),
    "denormals_are_zero": (
        "static float bf16_to_f32(uint16_t b)\n{\n    uint32_t u = (uint32_t)b << 16;",
        "static float bf16_to_f32(uint16_t b)\n{\n"
        "    uint32_t u = (b & 0x7F80u) ? (uint32_t)b << 16 : (uint32_t)(b & 0x8000u) << 16;"),
    "ties_away_from_zero": (
        "    double n = nearbyint(a / quantum);",
        "    double n = round(a / quantum);"),
    "no_key_rmsnorm": (
        "        z[s] = rstd * qdot;",
        "        z[s] = qdot; (void)rstd;"),
    "key_norm_sum_not_mean": (
        "        double rstd = 1.0 / sqrt(sumsq / (double)H + eps);\n        z[s]",
        "        double rstd = 1.0 / sqrt(sumsq + eps);\n        z[s]"),
    "softmax_sign_flipped": (
        "        z[s] = exp(z[s] - zmax);",
        "        z[s] = exp(zmax - z[s]);"),
    "no_max_subtraction": (
        "        z[s] = exp(z[s] - zmax);",
        "        z[s] = exp(z[s]); (void)zmax;"),
    "normalised_values_mixed": (
        "        z[s] = rstd * qdot;",
        "        z[s] = rstd * qdot;\n"
        "        for (int64_t hh = 0; hh < H; ++hh) ((double*)ks)[hh] *= rstd;"),
    "unrounded_prefix_mixed": (
        "        k[(int64_t)N * H + h] = oracle_bf16_to_f64(out_prefix[h]);",
        "    {   uint16_t t2 = add2 ? oracle_bf16_add(add[h], add2[h]) : add[h];\n"
        "        k[(int64_t)N * H + h] = (double)(bf16_to_f32(prefix[h]) + bf16_to_f32(t2)); }"),
    "prefix_left_out_of_mix": (
        "    for (int s = 0; s < S; ++s) {\n        z[s] = z[s] / denom;",
        "    z[N] = 0.0; denom = 0.0; for (int s = 0; s < N; ++s) denom += z[s];\n"
        "    if (N == 0) { z[0] = 1.0; denom = 1.0; }\n"
        "    for (int s = 0; s < S; ++s) {\n        z[s] = z[s] / denom;"),
    "final_eps_outside_sqrt": (
        "    double rstd = 1.0 / sqrt(sumsq / (double)H + eps);\n    for",
        "    double rstd = 1.0 / (sqrt(sumsq / (double)H) + eps);\n    for"),
    "final_sqrt_missing": (
        "    double rstd = 1.0 / sqrt(sumsq / (double)H + eps);\n    for",
        "    double rstd = 1.0 / (sumsq / (double)H + eps);\n    for"),
    "mixture_output_reports_prefix": (
        "            out_mix[h] = oracle_round_bf16(x); /* the pre-norm mixture, rounded once */",
        "            out_mix[h] = oracle_round_bf16(k[(int64_t)N * H + h]);"),
    "mixture_output_scaled": (
        "            out_mix_f64[h] = x;",
        "            out_mix_f64[h] = x * 1.0000001;"),
    "gamma_dropped": (
        "* rstd * oracle_bf16_to_f64(gamma[h]);",
        "* rstd;"),
    "gamma_as_offset": (
        "* rstd * oracle_bf16_to_f64(gamma[h]);",
        "* rstd * (1.0 + oracle_bf16_to_f64(gamma[h]));"),
    "snapshot_row_not_offset": (
        "            rows[s] = snapshots[s] + off;",
        "            rows[s] = snapshots[s];"),
    # the key RMSNorm and the logits: eps, weight, temperature
    "key_eps_dropped": (
        "        double rstd = 1.0 / sqrt(sumsq / (double)H + eps);\n        z[s]",
        "        double rstd = 1.0 / sqrt(sumsq / (double)H);\n        z[s]"),
    "key_eps_outside_sqrt": (
        "        double rstd = 1.0 / sqrt(sumsq / (double)H + eps);\n        z[s]",
        "        double rstd = 1.0 / (sqrt(sumsq / (double)H) + eps);\n        z[s]"),
    "query_times_gamma": (
        "            qdot += oracle_bf16_to_f64(query[h]) * ks[h];",
        "            qdot += oracle_bf16_to_f64(query[h]) * oracle_bf16_to_f64(gamma[h]) * ks[h];"),
    "key_norm_weighted_by_gamma": (
        "            sumsq += ks[h] * ks[h];",
        "            sumsq += ks[h] * ks[h] * oracle_bf16_to_f64(gamma[h]) * oracle_bf16_to_f64(gamma[h]);"),
    "logit_temperature": (
        "        z[s] = rstd * qdot;",
        "        z[s] = rstd * qdot / sqrt((double)H);"),
    "final_eps_dropped": (
        "    double rstd = 1.0 / sqrt(sumsq / (double)H + eps);\n    for",
        "    double rstd = 1.0 / sqrt(sumsq / (double)H);\n    for"),
    "final_norm_sum_not_mean": (
        "    double rstd = 1.0 / sqrt(sumsq / (double)H + eps);\n    for",
        "    double rstd = 1.0 / sqrt(sumsq + eps);\n    for"),
}

# A pin that compares the oracle with itself at a tolerance (the output under a
# permutation of the snapshots) may fail for a mutant by accident, on a
# near-zero element; it does not count as catching one.
NOT_A_PIN = {"check_snapshot_permutation"}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, "mutation anchor for %s not unique/present" % name
    src = os.path.join(str(mutant_dir), name + ".c")
    with open(src, "w") as fh:
        fh.write(SRC.replace(old, new))
    lib = obuild.build(source=src, output=os.path.join(str(mutant_dir), "lib%s.so" % name))
    orc = oracle.Oracle(lib)
    caught = []
    for check in pins.QUICK + [pins.check_round_vs_fractions]:
        if check.__name__ in NOT_A_PIN:
            continue
        try:
            check(orc)
        except (AssertionError, RuntimeError, FloatingPointError) as exc:
            caught.append((check.__name__, str(exc)[:200]))
            break
    assert caught, "mutant %s passed every pin" % name
    print("mutant", name, "caught by", caught[0][0])


# Mistakes in the mixing formula, the key RMSNorm, the softmax, the final
# RMSNorm or the mixture output: the exact tiny-H evaluation alone (rational and
# 60-digit arithmetic, no binary64) must catch each of them.
EXACT_ALONE = sorted(n for n in MUTANTS if n not in (
    "denormals_are_zero", "flush_to_zero",  # no subnormal sums in its cases: the golden examples pin these
    "no_max_subtraction",                    # logits O(1) there: the dominant-logit pin pins this
    "snapshot_row_not_offset",               # one token per call there: the permutation pins pin this
))


@pytest.mark.parametrize("name", EXACT_ALONE)
def test_exact_tiny_h_alone(name, mutant_dir):
    old, new = MUTANTS[name]
    src = os.path.join(str(mutant_dir), "exact_" + name + ".c")
    with open(src, "w") as fh:
        fh.write(SRC.replace(old, new))
    lib = obuild.build(source=src, output=os.path.join(str(mutant_dir), "libexact_%s.so" % name))
    with pytest.raises(AssertionError):
        pins.check_exact_tiny_h(oracle.Oracle(lib))
