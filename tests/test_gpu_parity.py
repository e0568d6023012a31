"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

out_prefix must be bit-exact and out_norm within 2 bf16 ulps or 1e-2 (see
parity.py), for the named workloads, every source count, ragged and extreme
sizes, both kernels (workgroup per token "W", split hidden "S") and their
vector widths.  Also: two addends == one pre-summed addend bitwise (page
"[#20545][perf] Kimi K3: fold the MoE-tail additions ...", section "Test
Coverage"), the hand-derived subnormal examples, determinism, HIP-graph
replay, canaries around the outputs, and the standalone add kernel.
"""
import os
import sys

import numpy as np
import pytest

import parity as P
import pins
from attention_residual_rmsnorm_amd import workloads as W

pytestmark = pytest.mark.gpu

# (variant, param): 0 = automatic; W = workgroup per token with param vectors
# per thread; S = split hidden with param waves per workgroup
VARIANTS = [(0, 0), (1, 1), (1, 2), (2, 1), (2, 2), (2, 7), (3, 0), (3, 4)]
VID = ["auto", "W1", "W2", "S1w", "S2w", "S7w", "hybrid", "hybrid4w"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def ar():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import attention_residual_rmsnorm_amd as ar

    ar.library()
    ar.attnres_init()
    yield ar
    ar.attnres_set_variant(0, 0)


@pytest.fixture
def variant(request, ar):
    v, param = request.param
    ar.attnres_set_variant(v, param)
    yield (v, param)
    ar.attnres_set_variant(0, 0)


def supported(ar, M, N, H):
    try:
        ar.attnres_plan(M, N, H)
        return True
    except ar.AttnResError:
        return False


_case_cache = {}


def case_for(key, fn):
    if key not in _case_cache:
        _case_cache[key] = fn()
    return _case_cache[key]


# --- the named workloads ------------------------------------------------------

@pytest.mark.parametrize("variant", VARIANTS, ids=VID, indirect=True)
@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_named_workload(ar, orc, variant, name):
    case = case_for(name, lambda: W.config_case(name))
    if not supported(ar, case.M, case.N, case.H):
        pytest.skip("variant not available for this size")
    say("case", name, "variant", variant, ar.attnres_plan(case.M, case.N, case.H))
    gp, gn = P.run_gpu(case)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(gp, gn, rp, rn, name)


def test_named_workload_structure():
    """The subnormal workload really plants subnormal sums and prefixes."""
    c = W.config_case("cfg3")
    sub = lambda b: ((b & 0x7F80) == 0) & ((b & 0x7F) != 0)
    assert sub(c.prefix).mean() > 0.009
    t = pins.bits_of(pins.tbf(c.add) + pins.tbf(c.add2))
    assert sub(t).mean() > 0.009


# --- how far inside the bar -------------------------------------------------------

@pytest.mark.parametrize("name", list(W.CONFIGS) + ["m256_n12"])
def test_error_margin(ar, orc, name):
    """How far inside the bar: the GPU's out_norm against the oracle's binary64
    value before its final rounding.  The binary32 arithmetic leaves an error
    that is absolute rather than relative (the logits' relative error of a few
    1e-6 moves the mixture by a few 1e-6, whatever the output's size), so two
    figures: for |value| >= 0.1 the error in bf16 ulps of the value (rounding
    alone accounts for up to 1/2) must stay within 0.75 ulp, and everywhere the
    error beyond half an ulp of rounding must stay below 1e-4 (the contract
    allows 2 ulps against the rounded oracle, or 1e-2)."""
    if name == "m256_n12":
        case = case_for(name, lambda: W.make_case(cfg=65, M=256, N=12, add2=True))
    else:
        case = case_for(name, lambda: W.config_case(name))
    gp, gn = P.run_gpu(case)
    _, _, exact = orc.fwd(case.prefix, case.add, case.add2, case.snapshots, case.query, case.gamma, case.eps,
                          want_f64=True)
    got = W.bf16_bits_to_f32(gn).astype(np.float64)
    nz = exact != 0
    ulp = np.where(nz, np.exp2(np.floor(np.log2(np.abs(np.where(nz, exact, 1.0)))) - 7), 2.0 ** -133)
    err_ulp = np.abs(got - exact) / ulp
    beyond = np.maximum(np.abs(got - exact) - ulp / 2, 0.0)
    big = np.abs(exact) >= 0.1
    say("error margin", name, ar.attnres_plan(case.M, case.N, case.H),
        "|v| >= 0.1: max %.4f ulp, mean %.4f; beyond rounding: max %.2e, at |v| %.3g (%.3f ulp)"
        % (err_ulp[big].max(), err_ulp[big].mean(), beyond.max(), abs(exact.flat[beyond.argmax()]),
           err_ulp.flat[beyond.argmax()]))
    assert err_ulp[big].max() <= 0.75, "%s: %.3f ulp" % (name, err_ulp[big].max())
    assert beyond.max() <= 1e-4, "%s: %.2e beyond rounding" % (name, beyond.max())


# --- two addends == one pre-summed addend, bitwise, N = 0..12 -----------------

@pytest.mark.parametrize("variant", [(1, 0), (2, 0)], ids=["W", "S"], indirect=True)
@pytest.mark.parametrize("M", [1, 8, 16, 32])
def test_add2_equals_presummed(ar, variant, M):
    for N in range(13):
        case = case_for(("presum", M, N), lambda: W.make_case(cfg=50, M=M, N=N, add2=True))
        t = pins.bits_of(pins.tbf(case.add) + pins.tbf(case.add2))
        a = P.run_gpu(case)
        import dataclasses

        b = P.run_gpu(dataclasses.replace(case, add=t, add2=None))
        assert np.array_equal(a[0], b[0]), "M=%d N=%d out_prefix" % (M, N)
        assert np.array_equal(a[1], b[1]), "M=%d N=%d out_norm" % (M, N)
        want = pins.torch_prefix(case.prefix, case.add, case.add2)
        assert np.array_equal(a[0], want), "M=%d N=%d prefix != torch" % (M, N)


# --- hand-derived fold-add examples through the kernels ----------------------

@pytest.mark.parametrize("variant", VARIANTS, ids=VID, indirect=True)
def test_golden_fold_add(ar, variant):
    rows = pins.read_golden_fold()
    H = 64 if variant[0] != 3 else 7168  # the hybrid serves rows of 4104..8192 elements
    M = len(rows)
    if not supported(ar, M, 0, H):
        pytest.skip("variant not available for this size")
    prefix = np.array([[r[0]] * H for r in rows], np.uint16)
    add = np.array([[r[1]] * H for r in rows], np.uint16)
    add2_rows = [r for r in rows if r[2] is not None]
    q = np.zeros(H, np.uint16)
    g = np.full(H, 0x3F80, np.uint16)
    # rows with add2
    idx = [i for i, r in enumerate(rows) if r[2] is not None]
    c = W.Case("golden", len(idx), H, prefix[idx], add[idx], np.array([[r[2]] * H for r in add2_rows], np.uint16),
               [], q, g)
    gp, _ = P.run_gpu(c)
    for k, i in enumerate(idx):
        assert np.all(gp[k] == rows[i][3]), "row %d: %04x != %04x" % (i, gp[k][0], rows[i][3])
    idx1 = [i for i, r in enumerate(rows) if r[2] is None]
    c1 = W.Case("golden1", len(idx1), H, prefix[idx1], add[idx1], None, [], q, g)
    gp1, _ = P.run_gpu(c1)
    for k, i in enumerate(idx1):
        assert np.all(gp1[k] == rows[i][3])


@pytest.mark.parametrize("variant", [(1, 0), (2, 0)], ids=["W", "S"], indirect=True)
@pytest.mark.parametrize("add2", [True, False], ids=["add2", "no_add2"])
def test_fold_every_bit_pattern(ar, orc, variant, add2):
    """out_prefix is bit-exact for every input, special values included: each of
    prefix, add and add2 holds every bf16 bit pattern once (NaN, +-Inf,
    subnormals, +-0, sums that overflow to Inf), at different offsets, against
    the oracle's two tensor additions; a NaN result only has to be a NaN.
    (out_norm is outside the parity contract for non-finite inputs.)"""
    import dataclasses

    M, H = 10, 7168
    rng = np.random.default_rng(91)
    every = np.arange(1 << 16, dtype=np.uint16)

    def field(shift):
        v = rng.integers(0, 1 << 16, M * H).astype(np.uint16)
        v[:1 << 16] = np.roll(every, shift)
        return v.reshape(M, H)

    prefix, add, add2v = field(0), field(12345), field(40000)
    base = case_for(("fold-bits",), lambda: W.make_case(cfg=64, M=M, N=2, add2=True))
    case = dataclasses.replace(base, prefix=prefix, add=add, add2=add2v if add2 else None)
    say("fold bit patterns", variant, add2, ar.attnres_plan(M, 2, H))
    gp, _ = P.run_gpu(case)
    t = orc.add_tensor(add.ravel(), add2v.ravel()) if add2 else add.ravel()
    want = orc.add_tensor(prefix.ravel(), t).reshape(M, H)
    nan = P.is_nan16(want)
    assert np.array_equal(gp[~nan], want[~nan]), "out_prefix differs at %d places" % int((gp[~nan] != want[~nan]).sum())
    assert np.all(P.is_nan16(gp[nan]))


def _cancelling_case(N, noise=1e-3, M=3, H=7168, seed=5):
    """Zero query (every logit 0, equal weights), p' = -snap_0 + noise, the
    further snapshots in exactly opposite pairs and, if one is left, one of the
    noise's size: the mixture is about `noise` of its terms."""
    rng = np.random.default_rng(seed)
    bf = lambda x: W.to_bf16_bits(np.asarray(x, np.float64))
    f = lambda b: W.bf16_bits_to_f32(b).astype(np.float64)
    s0 = bf(rng.standard_normal((M, H)))
    snaps = [s0]
    while N - len(snaps) >= 2:
        s = bf(rng.standard_normal((M, H)))
        snaps += [s, s ^ np.uint16(0x8000)]
    if len(snaps) < N:
        snaps.append(bf(noise * rng.standard_normal((M, H))))
    assert len(snaps) == N
    prefix = bf(-f(s0) + noise * rng.standard_normal((M, H)))
    add = np.zeros((M, H), np.uint16)
    gamma = bf(1.0 + 0.1 * rng.standard_normal(H))
    return W.Case("cancelling", M, H, prefix, add, None, snaps, np.zeros(H, np.uint16), gamma)


@pytest.mark.parametrize("variant", [(0, 0), (2, 1), (2, 2), (2, 7)], ids=["auto", "S1w", "S2w", "S7w"],
                         indirect=True)
@pytest.mark.parametrize("noise", [1e-3, 0.15, 0.3, 0.6])
@pytest.mark.parametrize("N", [1, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12])
def test_cancelling_sources(ar, orc, variant, N, noise):
    """Sources that nearly cancel.  The split kernel takes sum x^2 = alpha' G
    alpha from its one exchange for few sources.  With noise 1e-3 that form
    would lose most of sum x^2 to cancellation, so the kernel must detect it
    and run the second exchange; with 0.15 the conditioning bound still sends
    it there; with 0.6 (and 0.3 at N = 1) the sources cancel by a factor of
    about 12 to 57, under the bound, so the form is accepted and its rounding
    must stay far below the tolerance.  From 6 snapshots (two exchanges) the
    second exchange sums the chunks' x^2 of the cancelled mixture.  out_norm
    within the parity bound of the oracle either way."""
    if not supported(ar, 3, N, 7168):
        pytest.skip("variant not available for this size")
    case = case_for(("cancel", N, noise), lambda: _cancelling_case(N, noise))
    say("cancelling sources", N, noise, variant, ar.attnres_plan(case.M, N, case.H))
    gp, gn = P.run_gpu(case)
    rp, rn = P.run_oracle(orc, case)
    x = np.abs(W.bf16_bits_to_f32(rn)).max()
    assert x > 0.1, "the case must give a non-trivial normalised mixture"
    P.assert_parity(gp, gn, rp, rn, "cancelling N=%d" % N)


# --- ragged, tiny and maximal shapes -----------------------------------------

SHAPES = [
    (1, 8, 0), (3, 8, 12), (2, 64, 1), (5, 520, 3), (3, 1000, 12), (67, 1000, 5),
    (4, 4104, 7), (2, 7176, 12), (9, 8192, 12), (2, 8200, 4), (3, 16384, 12), (1, 16384, 0),
    (65, 7168, 2), (130, 512, 12),
]


@pytest.mark.parametrize("variant", VARIANTS, ids=VID, indirect=True)
@pytest.mark.parametrize("M,H,N", SHAPES)
def test_shapes(ar, orc, variant, M, H, N):
    if not supported(ar, M, N, H):
        pytest.skip("variant not available for this size")
    case = case_for(("shape", M, H, N), lambda: W.make_case(cfg=60, M=M, H=H, N=N, add2=(N % 2 == 0)))
    say("shape", M, H, N, "variant", variant, ar.attnres_plan(M, N, H))
    gp, gn = P.run_gpu(case)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(gp, gn, rp, rn, "M=%d H=%d N=%d" % (M, H, N))


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 8, 9, 12])
@pytest.mark.parametrize("M", [1, 2, 8, 9, 16, 24, 32, 40, 41, 48, 49, 56, 57, 64, 65, 88, 89, 96, 97])
def test_dispatch_boundaries(ar, orc, M, N):
    """The automatic dispatch on both sides of each of its token-count bounds
    (for N >= 6, two exchanges: 1-wave chunks up to 48 tokens, up to 64 with
    at most 8 snapshots, else 4-wave up to 64, 1-wave again up to 88, then
    2-wave up to 96 from 8 snapshots on and 1-wave at N = 7; for 2 <= N <= 5,
    the one-exchange form, 1-wave chunks up to 40 / 56 / 64 tokens at N = 2 /
    3 / 4-5, up to 8 at N = 1; then a workgroup per token) and source-count
    bounds (the split
    kernel's single-exchange form up to five snapshots, 1-wave chunks at 49-64
    tokens up to 8, and the halved polling of up to 32 values; one group of
    up to four sources in kernel W)."""
    case = case_for(("bound", M, N), lambda: W.make_case(cfg=62, M=M, N=N, add2=(M % 2 == 0)))
    say("boundary", M, N, ar.attnres_plan(M, N, case.H))
    gp, gn = P.run_gpu(case)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(gp, gn, rp, rn, "M=%d N=%d" % (M, N))


@pytest.mark.parametrize("N", [0, 1, 3, 4, 7, 8, 12])
@pytest.mark.parametrize("M", [256, 257, 264, 288, 289, 319, 320, 321, 336, 352, 353, 383, 384, 385, 511])
def test_hybrid_boundaries(ar, orc, M, N):
    """Past the CU count: the automatic dispatch's hybrid launch (kernel W on
    the first 256 tokens, 1-, 2- or 4-wave split chunks or half rows on the
    rest) at its bounds, and kernel W beyond it (two tokens on some CUs),
    every output element against the oracle."""
    case = case_for(("hybrid", M, N), lambda: W.make_case(cfg=67, M=M, N=N, add2=(N % 2 == 0)))
    say("hybrid", M, N, ar.attnres_plan(M, N, case.H))
    gp, gn = P.run_gpu(case)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(gp, gn, rp, rn, "M=%d N=%d" % (M, N))


@pytest.mark.parametrize("H", [8192, 4104])
@pytest.mark.parametrize("N", [4, 12])
@pytest.mark.parametrize("M", [300, 352])
def test_hybrid_other_widths(ar, orc, M, N, H):
    """The hybrid launch on rows of 1,024 and 513 vectors, whose workgroups
    are 512 and 320 threads wide (automatic at H = 8192, forced at 4104, where
    the automatic dispatch takes other kernels): 4- or 2-wave chunks at 300
    tokens, half-row chunks (8 and 5 waves) at 352, against the oracle."""
    case = case_for(("hybridw", M, N, H), lambda: W.make_case(cfg=66, M=M, H=H, N=N, add2=(N % 2 == 0)))
    try:
        if H == 4104:
            ar.attnres_set_variant(3, 0)
        plan = ar.attnres_plan(M, N, H)
        say("hybrid widths", M, N, H, plan)
        assert plan[0] == 3 and (M < 352 or plan[1] == 2)
        gp, gn = P.run_gpu(case)
    finally:
        ar.attnres_set_variant(0, 0)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(gp, gn, rp, rn, "M=%d N=%d H=%d" % (M, N, H))


# (M, H, N): kernel W's single-group form (rows of at most 256 vectors, up to
# 131072 threads per call) on both sides of its bound, ragged short rows, and
# the split bounds for rows of 257..895 vectors (1-wave chunks up to 32 / 48 /
# 64 / 96 tokens at N = 4 / 5-7 / 8-11 / 12); H = 896 is a tensor-parallel
# rank's share (1/8) of 7168
SHORT_ROWS = [(1, 896, n) for n in (0, 1, 3, 4, 5, 8, 12)] + [
    (7, 904, 2), (7, 904, 5), (7, 904, 12), (1024, 896, 12), (1025, 896, 12), (512, 2048, 8), (513, 2048, 8),
    (33, 2048, 12), (1, 3584, 12), (32, 3584, 8), (33, 3584, 12), (65, 3584, 12), (96, 4096, 12), (97, 3584, 12),
    (80, 3584, 8), (3, 4096, 7), (1, 3584, 3), (32, 3584, 4), (33, 4096, 4), (48, 4096, 5), (49, 3584, 7),
    (64, 3584, 8), (65, 4096, 11)]


@pytest.mark.parametrize("H", [16384, 12288])
@pytest.mark.parametrize("N", [0, 4, 12])
@pytest.mark.parametrize("M", [1, 16, 17, 32, 33, 48, 49, 96, 97])
def test_very_long_rows_dispatch(ar, orc, M, H, N):
    """Rows longer than 8192 under the automatic dispatch, on both sides of
    each token bound (2-wave split chunks up to 16 tokens and from 33 to 48,
    4-wave from 17 to 32 and 49 to 96, then kernel W)."""
    case = case_for(("vlong", M, H, N), lambda: W.make_case(cfg=69, M=M, H=H, N=N, add2=(M % 2 == 1)))
    say("very long rows", M, H, N, ar.attnres_plan(M, N, H))
    gp, gn = P.run_gpu(case)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(gp, gn, rp, rn, "M=%d H=%d N=%d" % (M, H, N))


@pytest.mark.parametrize("M,H,N", SHORT_ROWS)
def test_short_rows(ar, orc, M, H, N):
    """Rows shorter than 7168 under the automatic dispatch."""
    case = case_for(("short", M, H, N), lambda: W.make_case(cfg=63, M=M, H=H, N=N, add2=(M % 2 == 1)))
    say("short rows", M, H, N, ar.attnres_plan(M, N, H))
    gp, gn = P.run_gpu(case)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(gp, gn, rp, rn, "M=%d H=%d N=%d" % (M, H, N))


def test_short_rows_deterministic(ar):
    """The single-group form's sums run in a fixed order: same bits every call."""
    case = case_for(("short-det", 512, 896, 12), lambda: W.make_case(cfg=63, M=512, H=896, N=12, add2=True))
    first = P.run_gpu(case)
    for _ in range(10):
        again = P.run_gpu(case)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])


def _random_cases(n=80, seed=2026):
    rng = np.random.default_rng(seed)
    variants = VARIANTS + [(1, 4), (2, 4), (2, 8)]
    out = []
    while len(out) < n:
        H = int(rng.choice([8, 16, 64, 520, 896, 904, 1000, 2048, 3584, 4104, 7168, 7176, 8192, 8200, 12000,
                            16384]))
        M = int(rng.integers(1, 81))
        if M * H > 400_000:
            continue
        N = int(rng.integers(0, 13)) if rng.random() < 0.8 else int(rng.integers(13, 32))
        cancel = bool(N >= 1 and rng.random() < 0.1)
        out.append((M, H, N, bool(rng.random() < 0.7), variants[int(rng.integers(0, len(variants)))], cancel))
    return out


@pytest.mark.parametrize("M,H,N,add2,var,cancel", _random_cases())
def test_random_shapes(ar, orc, M, H, N, add2, var, cancel):
    """Seeded random token counts, hidden sizes (ragged tails, short rows
    included), source counts up to 31, with and without the second addend,
    under a random forced kernel variant (skipped where that variant cannot
    serve the size); about one case in ten has sources that nearly cancel."""
    ar.attnres_set_variant(*var)
    try:
        try:
            ar.attnres_plan(M, N, H)
        except ar.AttnResError:
            pytest.skip("variant not available for this size")
        if cancel:
            case = _cancelling_case(N, 0.15 if M % 2 else 1e-3, M=M, H=H, seed=M * 131 + N)
        else:
            case = W.make_case(cfg=66, M=M, H=H, N=N, add2=add2)
        say("random", M, H, N, add2, var, cancel, ar.attnres_plan(M, N, H))
        gp, gn = P.run_gpu(case)
    finally:
        ar.attnres_set_variant(0, 0)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(gp, gn, rp, rn, "M=%d H=%d N=%d add2=%s variant=%s cancel=%s" % (M, H, N, add2, var, cancel))


def test_beyond_split_slots_and_grid(ar, orc):
    """M above the split-hidden token slots (workgroup per token; 600 tokens put
    two workgroups on some CUs), the prefill-sized calls bench.py times (1,024
    tokens, N = 12) and the form with four vectors per thread (2,048 and
    4,096 tokens), and M above the W grid cap (grid-stride over tokens),
    checked on sampled rows."""
    import torch

    for M, H, N in ((600, 7168, 4), (1024, 7168, 12), (2048, 7168, 12), (4096, 8192, 4), ((1 << 20) + 5, 8, 2)):
        case = W.make_case(cfg=61, M=M, H=H, N=N, add2=True)
        say("large M", M, H, N, ar.attnres_plan(M, N, H))
        gp, gn = P.run_gpu(case)
        idx = np.unique(np.r_[0, 1, M // 2, M - 2, M - 1, np.random.default_rng(0).integers(0, M, 64)])
        sub = case.rows(idx)
        rp, rn = P.run_oracle(orc, sub)
        P.assert_parity(gp[idx], gn[idx], rp, rn, "M=%d" % M)
        del gp, gn
        torch.cuda.empty_cache()


def test_empty_batch(ar):
    import torch

    z = torch.empty((0, 7168), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(7168, dtype=torch.bfloat16, device="cuda")
    op, on = ar.attnres_add_rmsnorm_fwd(z, z, z, [z, z], v, v, 1e-6)
    assert op.shape == (0, 7168) and on.shape == (0, 7168)


@pytest.mark.parametrize("variant", [(1, 0), (2, 0)], ids=["W", "S"], indirect=True)
def test_in_place_prefix(ar, orc, variant):
    case = W.make_case(cfg=62, M=8, N=5, add2=True)
    prefix = P.dev(case.prefix)
    d = P.dev
    op, on = ar.attnres_add_rmsnorm_fwd(prefix, d(case.add), d(case.add2), [d(s) for s in case.snapshots],
                                        d(case.query), d(case.gamma), case.eps, out_prefix=prefix)
    assert op.data_ptr() == prefix.data_ptr()
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(P.host(op), P.host(on), rp, rn, "in place")


# --- determinism, graphs, canaries ---------------------------------------------

# W; split with 1, 2 (gather in every wave), 7 waves (wave 0); the hybrid of W and 4-wave chunks
SYNC_VARIANTS = [(1, 0), (2, 1), (2, 2), (2, 7), (3, 0), (3, 4)]
SYNC_VID = ["W", "S1w", "S2w", "S7w", "hybrid", "hybrid4w"]


@pytest.mark.parametrize("variant", SYNC_VARIANTS, ids=SYNC_VID, indirect=True)
@pytest.mark.parametrize("name", ["cfg4", "cfg2"])  # N = 12: two exchanges; N = 4: the Gram form's one
def test_deterministic(ar, variant, name):
    case = case_for(name, lambda: W.config_case(name))
    if not supported(ar, case.M, case.N, case.H):
        pytest.skip("variant not available for this size")
    first = P.run_gpu(case)
    for _ in range(20):
        again = P.run_gpu(case)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])


@pytest.mark.parametrize("variant", [(2, 1), (2, 2), (2, 7)], ids=["S1w", "S2w", "S7w"], indirect=True)
def test_exchange_forms_alternate(ar, orc, variant):
    """Calls with one exchange (the Gram form, N = 4), two exchanges (N = 8) and
    the Gram form's fallback (cancelling sources, N = 4) in turn on the same
    token slots: each form advances the per-token epoch at its own point, and
    every call must still see only its own records (same bits as its first
    run, within the bound of the oracle)."""
    cases = [W.make_case(cfg=75, M=8, N=4, add2=True), W.make_case(cfg=76, M=8, N=8, add2=True),
             _cancelling_case(4, 1e-3, M=8)]
    ar.attnres_debug_set_slot_rotation(False)  # every call on token slots 0..7
    try:
        first = [P.run_gpu(c) for c in cases]
        for c, (gp, gn) in zip(cases, first):
            rp, rn = P.run_oracle(orc, c)
            P.assert_parity(gp, gn, rp, rn, c.name)
        for rep in range(30):
            i = (rep * 7) % 3
            gp, gn = P.run_gpu(cases[i])
            assert np.array_equal(gp, first[i][0]) and np.array_equal(gn, first[i][1]), "call %d (case %d)" % (
                rep, i)
    finally:
        ar.attnres_debug_set_slot_rotation(True)
    assert ar.attnres_debug_timeouts() == 0


@pytest.mark.parametrize("variant", SYNC_VARIANTS, ids=SYNC_VID, indirect=True)
# the split kernel's two exchanges, its Gram form's one, and its two-wave form (40 snapshots)
@pytest.mark.parametrize("N", [8, 4, 40])
def test_graph_replay(ar, variant, N):
    """Capture one call into a HIP graph; replay it with fresh inputs copied
    in between (eager work and synchronisation between replays); every replay
    must equal the eager call on the same inputs, bit for bit."""
    import torch

    if not supported(ar, 16, N, 7168):
        pytest.skip("variant not available for this size")
    cases = [W.make_case(cfg=70 + i, M=16, N=N, add2=True) for i in range(4)]
    c0 = cases[0]
    d = P.dev
    ins = dict(prefix=d(c0.prefix), add=d(c0.add), add2=d(c0.add2), snaps=[d(s) for s in c0.snapshots],
               query=d(c0.query), gamma=d(c0.gamma))
    outp = torch.empty_like(ins["prefix"])
    outn = torch.empty_like(ins["prefix"])

    def call():
        ar.attnres_add_rmsnorm_fwd(ins["prefix"], ins["add"], ins["add2"], ins["snaps"], ins["query"],
                                   ins["gamma"], c0.eps, out_prefix=outp, out_norm=outn)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(12):
        c = cases[rep % len(cases)]
        ins["prefix"].copy_(d(c.prefix))
        ins["add"].copy_(d(c.add))
        ins["add2"].copy_(d(c.add2))
        for t, src in zip(ins["snaps"], c.snapshots):
            t.copy_(d(src))
        ins["query"].copy_(d(c.query))
        ins["gamma"].copy_(d(c.gamma))
        outp.zero_()
        outn.zero_()
        g.replay()
        torch.cuda.synchronize()
        gp, gn = P.host(outp), P.host(outn)
        ep, en = P.run_gpu(c)
        assert np.array_equal(gp, ep) and np.array_equal(gn, en), "replay %d" % rep
    assert ar.attnres_debug_timeouts() == 0


@pytest.mark.parametrize("variant", [(1, 0), (2, 0), (3, 0), (3, 4)], ids=["W", "S", "hybrid", "hybrid4w"],
                         indirect=True)
def test_canaries(ar, orc, variant):
    """Outputs live inside larger buffers filled with a canary pattern: nothing
    outside [M,H] may change."""
    import torch

    case = W.make_case(cfg=63, M=7, H=1000, N=3, add2=True) if variant[0] != 3 else \
        W.make_case(cfg=63, M=21, H=7176, N=3, add2=True)
    n = case.M * case.H
    pad = 4096
    canary = 0x7E57
    bufp = torch.full((n + 2 * pad,), canary, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    bufn = torch.full((n + 2 * pad,), canary, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    outp = bufp[pad:pad + n].view(case.M, case.H)
    outn = bufn[pad:pad + n].view(case.M, case.H)
    gp, gn = P.run_gpu(case, out_prefix=outp, out_norm=outn)
    for buf in (bufp, bufn):
        h = P.host(buf)
        assert np.all(h[:pad] == canary) and np.all(h[pad + n:] == canary)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(gp, gn, rp, rn, "canary")


def test_no_barrier_timeouts(ar):
    assert ar.attnres_debug_timeouts() == 0


def test_bounded_waits_give_up(ar, orc):
    """The split kernel's waits at its per-token barriers are bounded.  With
    the spin limit forced down to one re-poll from the host, calls of both
    exchange forms and of the two-wave form (32..63 snapshots) still finish and the waits that give up are counted; each
    such call, run on a cleared scratch, leaves out_prefix exact and every
    out_norm element either within the bar of the oracle or NaN (a wait that
    gives up takes NaN for what it did not receive).  Once the scratch is
    cleared and the limit restored, calls are exact again."""
    import torch

    two = case_for("cfg4", lambda: W.config_case("cfg4"))  # two exchanges
    one = case_for("cfg2", lambda: W.config_case("cfg2"))  # the Gram form's one
    many = W.make_case(cfg=87, M=3, N=40, add2=True)      # the two-wave form's two record pages
    refs = [P.run_oracle(orc, c) for c in (two, one, many)]
    forced = 0
    nan_seen = 0
    ar.attnres_set_variant(2, 1)
    try:
        for rep in range(6):
            for case, (rp, rn) in zip((two, one, many), refs):
                ar.attnres_debug_reset_scratch()
                ar.attnres_debug_set_spin_limit(1)
                try:
                    gp, gn = P.run_gpu(case)
                    torch.cuda.synchronize()
                finally:
                    ar.attnres_debug_set_spin_limit(0)
                forced += ar.attnres_debug_timeouts()
                assert np.array_equal(gp, rp), "out_prefix depends on no exchange"
                nan = P.is_nan16(gn)
                nan_seen += int(nan.sum())
                bad = P.norm_mismatches(gn, rn) & ~nan
                assert not bad.any(), "call %d M=%d N=%d: %d elements neither exact nor NaN" % (
                    rep, case.M, case.N, int(bad.sum()))
    finally:
        ar.attnres_debug_set_spin_limit(0)
        ar.attnres_debug_reset_scratch()
        ar.attnres_set_variant(0, 0)
    say("forced timeouts", forced, "NaN elements", nan_seen)
    assert forced > 0
    assert ar.attnres_debug_timeouts() == 0
    for case in (two, one, many):
        gp, gn = P.run_gpu(case)
        rp, rn = P.run_oracle(orc, case)
        P.assert_parity(gp, gn, rp, rn, "after the reset")
    assert ar.attnres_debug_timeouts() == 0


# (forced variant, case): kernel S's two exchanges (1 and 7 waves per chunk),
# its Gram form, the automatic single-token call (14 one-wave chunks), the
# hybrid's split part, and the two- and four-wave forms at 40 snapshots (both
# record pages)
EXCHANGE_CASES = [((2, 1), "cfg4"), ((2, 7), "cfg4"), ((2, 2), "cfg2"), ((0, 0), "cfg4b"), ((3, 0), "hybrid21"),
                  ((0, 0), "twowave40"), ((2, 4), "twowave40")]


@pytest.mark.parametrize("mode", [1, 2], ids=["device-copies", "chunks-on-other-XCDs"])
def test_exchange_copies(ar, orc, mode):
    """The exchange's two copies of every record: the device-scope copies read
    alone (mode 1), and the chunks of each token placed on different XCDs, so
    that their L2 copies stay unseen and every wait falls back to the
    device-scope copies (mode 2).  Each call against the default mode's bits
    and against the oracle, with no wait given up."""
    import torch

    for variant, name in EXCHANGE_CASES:
        if name == "hybrid21":
            case = case_for(name, lambda: W.make_case(cfg=68, M=21, H=7176, N=12, add2=True))
        elif name == "twowave40":
            case = case_for(name, lambda: W.make_case(cfg=69, M=9, N=40, add2=True))
        else:
            case = case_for(name, lambda: W.config_case(name))
        ar.attnres_set_variant(*variant)
        try:
            say("exchange mode", mode, variant, name, ar.attnres_plan(case.M, case.N, case.H))
            ep, en = P.run_gpu(case)
            ar.attnres_debug_set_exchange(mode)
            try:
                gp, gn = P.run_gpu(case)
                torch.cuda.synchronize()
            finally:
                ar.attnres_debug_set_exchange(0)
        finally:
            ar.attnres_set_variant(0, 0)
        assert np.array_equal(gp, ep) and np.array_equal(gn, en), "%s %s: modes differ" % (variant, name)
        rp, rn = P.run_oracle(orc, case)
        P.assert_parity(gp, gn, rp, rn, "mode %d %s %s" % (mode, variant, name))
    assert ar.attnres_debug_timeouts() == 0


EPOCH_PERIOD = 0x7FFFFFFF


def test_epoch_wrap(ar, orc):
    """The split kernel's per-token epoch wraps from 2^31 - 2 to 0, and the
    wrapping call clears the records it does not read (here: of the chunk
    indices it does not use).
    A call with 14 chunks (one wave each) at epoch 5 leaves records at chunk
    indices 7..13; calls with 7 chunks (two waves each) then run across the
    wrap; another 14-chunk call on different inputs at epoch 5 again expects
    the tags those old records carry, and must still be exact, because the
    wrapping call cleared them.  Epochs are set from the host between calls."""
    a = case_for(("wrap", 0), lambda: W.make_case(cfg=80, M=8, N=8, add2=True))
    b = case_for(("wrap", 1), lambda: W.make_case(cfg=81, M=8, N=8, add2=True))
    ra, rb = P.run_oracle(orc, a), P.run_oracle(orc, b)
    try:
        ar.attnres_debug_reset_scratch()
        ar.attnres_debug_set_slot_rotation(False)  # every call on token slots 0..7
        ar.attnres_set_variant(2, 1)
        assert ar.attnres_plan(8, 8, 7168)[1] == 14
        ar.attnres_debug_set_epoch(5)
        P.assert_parity(*P.run_gpu(a), *ra, "14 chunks at epoch 5")
        ar.attnres_set_variant(2, 2)
        assert ar.attnres_plan(8, 8, 7168)[1] == 7
        ar.attnres_debug_set_epoch(EPOCH_PERIOD - 2)
        for i in range(4):  # epochs 2^31 - 3 .. 2^31 - 2, then 0 and 1
            say("wrap: 7-chunk call", i)
            P.assert_parity(*P.run_gpu(b), *rb, "7 chunks, call %d across the wrap" % i)
        ar.attnres_set_variant(2, 1)
        ar.attnres_debug_set_epoch(5)
        P.assert_parity(*P.run_gpu(b), *rb, "14 chunks at epoch 5 after the wrap")
        assert ar.attnres_debug_timeouts() == 0
        with pytest.raises(ar.AttnResError):
            ar.attnres_debug_set_epoch(EPOCH_PERIOD)
    finally:
        ar.attnres_set_variant(0, 0)
        ar.attnres_debug_set_slot_rotation(True)
        ar.attnres_debug_reset_scratch()


def test_bounded_waits_give_up_four_wave(ar, orc):
    """The same for the split kernel's four-wave form (40 snapshots, both
    record pages): with the spin limit forced down to one re-poll, every
    call finishes, the give-ups are counted, out_prefix stays exact and every
    out_norm element is exact or NaN; after a reset, exact again."""
    import torch

    case = W.make_case(cfg=88, M=3, N=40, add2=True)
    rp, rn = P.run_oracle(orc, case)
    forced = 0
    ar.attnres_set_variant(2, 4)
    try:
        assert ar.attnres_plan(case.M, case.N, case.H) == (2, 7, 256)
        for rep in range(4):
            ar.attnres_debug_reset_scratch()
            ar.attnres_debug_set_spin_limit(1)
            try:
                gp, gn = P.run_gpu(case)
                torch.cuda.synchronize()
            finally:
                ar.attnres_debug_set_spin_limit(0)
            forced += ar.attnres_debug_timeouts()
            assert np.array_equal(gp, rp), "out_prefix depends on no exchange"
            nan = P.is_nan16(gn)
            bad = P.norm_mismatches(gn, rn) & ~nan
            assert not bad.any(), "call %d: %d elements neither exact nor NaN" % (rep, int(bad.sum()))
        ar.attnres_debug_reset_scratch()
        assert forced > 0
        assert ar.attnres_debug_timeouts() == 0
        gp, gn = P.run_gpu(case)
        P.assert_parity(gp, gn, rp, rn, "after the reset")
        assert ar.attnres_debug_timeouts() == 0
    finally:
        ar.attnres_debug_set_spin_limit(0)
        ar.attnres_debug_reset_scratch()
        ar.attnres_set_variant(0, 0)


def test_epoch_wrap_value_slots(ar, orc):
    """Across the wrap with the same chunk count but fewer first-exchange
    values: a 31-snapshot call at epoch 5 fills all 64 value slots of chunk
    indices 0..13, 8-snapshot calls (18 values) run across the wrap, and a
    31-snapshot call on other inputs at epoch 5 must still be exact, because
    the wrapping call cleared value slots 18..63 as well."""
    a = case_for(("wrapv", 0), lambda: W.make_case(cfg=85, M=8, N=31, add2=True))
    b = case_for(("wrapv", 1), lambda: W.make_case(cfg=86, M=8, N=31, add2=False))
    c = case_for(("wrapv", 2), lambda: W.make_case(cfg=84, M=8, N=8, add2=True))
    ra, rb, rc = P.run_oracle(orc, a), P.run_oracle(orc, b), P.run_oracle(orc, c)
    try:
        ar.attnres_debug_reset_scratch()
        ar.attnres_debug_set_slot_rotation(False)
        ar.attnres_set_variant(2, 1)
        assert ar.attnres_plan(8, 31, 7168)[1] == 14 and ar.attnres_plan(8, 8, 7168)[1] == 14
        ar.attnres_debug_set_epoch(5)
        P.assert_parity(*P.run_gpu(a), *ra, "31 snapshots at epoch 5")
        ar.attnres_debug_set_epoch(EPOCH_PERIOD - 2)
        for i in range(4):
            say("wrap: 8-snapshot call", i)
            P.assert_parity(*P.run_gpu(c), *rc, "8 snapshots, call %d across the wrap" % i)
        ar.attnres_debug_set_epoch(5)
        P.assert_parity(*P.run_gpu(b), *rb, "31 snapshots at epoch 5 after the wrap")
        assert ar.attnres_debug_timeouts() == 0
    finally:
        ar.attnres_set_variant(0, 0)
        ar.attnres_debug_set_slot_rotation(True)
        ar.attnres_debug_reset_scratch()


@pytest.mark.parametrize("variant,shape", [((0, 0), (2, 14, 128)), ((2, 4), (2, 7, 256))],
                         ids=["two-wave", "four-wave"])
def test_epoch_wrap_two_wave(ar, orc, variant, shape):
    """The same across the wrap for the split kernel's two- and four-wave
    forms (32..63 snapshots), whose second record page sits at chunk indices
    16 and on: such a call at epoch 5 leaves records there, one-wave 14-chunk
    calls run across the wrap (the wrapping call clears indices 14..31), and
    a call of the same form on other inputs at epoch 5 again expects the tags
    the old page-1 records carry, and must still be exact."""
    a = case_for(("wrap2", 0), lambda: W.make_case(cfg=82, M=8, N=40, add2=True))
    b = case_for(("wrap2", 1), lambda: W.make_case(cfg=83, M=8, N=40, add2=False))
    c = case_for(("wrap2", 2), lambda: W.make_case(cfg=84, M=8, N=8, add2=True))
    ra, rb, rc = P.run_oracle(orc, a), P.run_oracle(orc, b), P.run_oracle(orc, c)
    try:
        ar.attnres_debug_reset_scratch()
        ar.attnres_debug_set_slot_rotation(False)  # every call on token slots 0..7
        ar.attnres_set_variant(*variant)
        assert ar.attnres_plan(8, 40, 7168) == shape
        ar.attnres_debug_set_epoch(5)
        P.assert_parity(*P.run_gpu(a), *ra, "two-wave call at epoch 5")
        ar.attnres_set_variant(2, 1)
        assert ar.attnres_plan(8, 8, 7168)[1] == 14
        ar.attnres_debug_set_epoch(EPOCH_PERIOD - 2)
        for i in range(4):  # epochs 2^31 - 3 .. 2^31 - 2, then 0 and 1
            say("wrap: one-wave call", i)
            P.assert_parity(*P.run_gpu(c), *rc, "14 one-wave chunks, call %d across the wrap" % i)
        ar.attnres_set_variant(*variant)
        ar.attnres_debug_set_epoch(5)
        P.assert_parity(*P.run_gpu(b), *rb, "two-wave call at epoch 5 after the wrap")
        assert ar.attnres_debug_timeouts() == 0
    finally:
        ar.attnres_set_variant(0, 0)
        ar.attnres_debug_set_slot_rotation(True)
        ar.attnres_debug_reset_scratch()


def test_concurrent_streams(ar, orc):
    """Split-kernel calls enqueued on two streams with no ordering between
    them (two exchanges and the Gram form's one, 1- and 2-wave chunks, the
    hybrid launch's 1- and 2-wave chunks, and the two- and four-wave forms'
    two record pages at 40 snapshots): each call takes its own token
    slots of the scratch, so calls that run at the same time do not share
    records.  Every output against the oracle, and no wait given up."""
    import torch

    cases = [W.make_case(cfg=90 + i, M=32, N=(12, 4, 8)[i % 3], add2=True) for i in range(6)]
    cases += [W.make_case(cfg=96, M=264, N=12, add2=True), W.make_case(cfg=97, M=288, N=4, add2=True),
              W.make_case(cfg=98, M=16, N=40, add2=True), W.make_case(cfg=99, M=4, H=16384, N=40, add2=True)]
    refs = [P.run_oracle(orc, c) for c in cases]
    d = P.dev
    ins = [(d(c.prefix), d(c.add), d(c.add2), [d(s) for s in c.snapshots], d(c.query), d(c.gamma)) for c in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    ar.attnres_debug_reset_scratch()  # slots from 0: the 20 calls take 504 of the 512
    outs = []
    for rep in range(2):
        for i, c in enumerate(cases):
            op, on = (torch.empty((c.M, c.H), dtype=torch.bfloat16, device="cuda") for _ in range(2))
            outs.append((i, op, on))
    torch.cuda.synchronize()
    for k, (i, op, on) in enumerate(outs):
        s = streams[k % 2]
        pre, add, add2, snaps, q, g = ins[i]
        ar.attnres_add_rmsnorm_fwd(pre, add, add2, snaps, q, g, cases[i].eps, out_prefix=op, out_norm=on,
                                   stream=s)
    torch.cuda.synchronize()
    say("concurrent streams", [ar.attnres_plan(c.M, c.N, c.H) for c in cases[:3] + cases[6:]])
    for k, (i, op, on) in enumerate(outs):
        P.assert_parity(P.host(op), P.host(on), *refs[i], "call %d (case %d, stream %d)" % (k, i, k % 2))
    assert ar.attnres_debug_timeouts() == 0


# --- the standalone add ----------------------------------------------------------

@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 4095, 65536, 65536 * 3 + 5])
def test_bf16_add(ar, orc, n):
    rng = np.random.default_rng(n)
    a = rng.integers(0, 1 << 16, n).astype(np.uint16)
    b = rng.integers(0, 1 << 16, n).astype(np.uint16)
    if n >= 65536:
        a[:65536] = np.arange(65536, dtype=np.uint16)  # every pattern once
    out = P.host(ar.attnres_bf16_add(P.dev(a), P.dev(b)))
    want = orc.add_tensor(a, b)
    nan = P.is_nan16(want)
    assert np.array_equal(out[~nan], want[~nan])
    assert np.all(P.is_nan16(out[nan]))


def test_single_hip_runtime(ar):
    """libattnres binds to the HIP runtime torch already loaded: exactly one
    libamdhip64 is mapped in the process."""
    maps = open("/proc/self/maps").read().splitlines()
    libs = sorted(set(l.split()[-1] for l in maps if "libamdhip64" in l))
    assert len(libs) == 1, libs
    assert any("libattnres.so" in l for l in maps)


def test_device_rounding_matches_definition(ar):
    """The hardware bf16 conversion behind every rounding in the kernels equals
    rounding by definition on all 2^32 binary32 inputs (NaN stays NaN)."""
    assert ar.attnres_selftest_rounding() == 0
