"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each ``check_*`` takes an ``oracle.Oracle`` (the real build or a planted
mutant) and raises ``AssertionError`` when the oracle disagrees with:

* worked IEEE examples derived by hand (``tests/golden/fold_add_worked.txt``),
* an independent library (PyTorch's CPU bf16 tensor additions),
* closed forms (a two-source softmax is a logistic function; q = 0 gives
  uniform weights; a single source gives the textbook RMSNorm),
* invariants (power-of-two scaling, token and source permutations),
* exact rounding computed with Python's ``fractions``.

None of them re-types the oracle's own loop: each compares against a
different route to the same value.  The checks are ordered cheap-first so a
mutant fails fast.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

from attention_residual_rmsnorm_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# helpers ------------------------------------------------------------------

def f64(bits) -> np.ndarray:
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def tbf(bits):
    """numpy bf16 bits -> torch bfloat16 CPU tensor (no copy of values)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def bits_of(t) -> np.ndarray:
    import torch

    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def torch_prefix(prefix, add, add2):
    """The unfused MoE tail: two (or one) PyTorch CPU bf16 tensor additions."""
    t = tbf(add) if add2 is None else tbf(add) + tbf(add2)
    return bits_of(tbf(prefix) + t)


def textbook_rmsnorm(x: np.ndarray, gamma_bits, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * gamma, rows of x in float64 (numpy)."""
    eps = float(np.float32(eps))
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * f64(gamma_bits)


def assert_close(got, want, rtol, atol=0.0, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    lim = atol + rtol * np.abs(want)
    bad = ~(err <= lim)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d mismatches, first at %s: got %r want %r"
                             % (what, int(bad.sum()), tuple(i), got[tuple(i)], want[tuple(i)]))


def scale_pow2(bits, k: int) -> np.ndarray:
    """Multiply bf16 values by 2^k by moving the exponent field (normal values
    only; zeros stay zero).  Exact by construction."""
    b = np.asarray(bits, np.uint16).astype(np.int32)
    e = (b >> 7) & 0xFF
    nz = e != 0
    assert np.all((e[nz] + k > 0) & (e[nz] + k < 255)), "scaling leaves the normal range"
    out = np.where(nz, (b & 0x807F) | ((e + k) << 7), b)
    return out.astype(np.uint16)


def rand_case(M, H, N, add2=True, seed=0):
    return W.make_case(cfg=900 + seed, M=M, H=H, N=N, add2=add2)


# fold-add ------------------------------------------------------------------

def read_golden_fold():
    rows = []
    with open(os.path.join(GOLDEN, "fold_add_worked.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            p, a, a2, want = line.split()
            rows.append((int(p, 16), int(a, 16), None if a2 == "-" else int(a2, 16), int(want, 16)))
    return rows


def check_golden_fold(orc):
    """Hand-derived IEEE examples, through the whole fused call (N=0, H=8)."""
    rows = read_golden_fold()
    assert len(rows) >= 9
    H = 8
    q = np.zeros(H, np.uint16)
    g = np.full(H, 0x3F80, np.uint16)
    for p, a, a2, want in rows:
        P = np.full((1, H), p, np.uint16)
        A = np.full((1, H), a, np.uint16)
        A2 = None if a2 is None else np.full((1, H), a2, np.uint16)
        out_prefix, _ = orc.fwd(P, A, A2, [], q, g, 1e-6)
        assert np.all(out_prefix == want), "fold %04x %04x %s: got %04x want %04x" % (
            p, a, a2, out_prefix[0, 0], want)


def check_prefix_vs_torch(orc):
    """Updated prefix == PyTorch CPU bf16 prefix + (routed + shared), and
    prefix + add without the second addend (library pin)."""
    for case in (rand_case(4, 1024, 1, add2=True, seed=1),
                 rand_case(3, 1024, 1, add2=False, seed=2),
                 W.make_case(cfg=903, M=4, H=2048, N=1, add2=True, special="subnormal")):
        out_prefix, _ = orc.fwd(case.prefix, case.add, case.add2, case.snapshots,
                                case.query, case.gamma, case.eps)
        want = torch_prefix(case.prefix, case.add, case.add2)
        bad = np.flatnonzero(out_prefix != want)
        assert bad.size == 0, "prefix differs from torch at %d places, first %d: %04x vs %04x" % (
            bad.size, bad[0], out_prefix.flat[bad[0]], want.flat[bad[0]])


def check_add2_equals_presummed(orc):
    """Two addends give bitwise the same updated prefix and output as one
    addend holding their bf16 sum (computed by PyTorch)."""
    for N in (0, 1, 5, 12):
        case = rand_case(3, 512, N, add2=True, seed=10 + N)
        t = bits_of(tbf(case.add) + tbf(case.add2))
        a = orc.fwd(case.prefix, case.add, case.add2, case.snapshots, case.query, case.gamma, case.eps)
        b = orc.fwd(case.prefix, t, None, case.snapshots, case.query, case.gamma, case.eps)
        assert np.array_equal(a[0], b[0]), "N=%d: out_prefix differs" % N
        assert np.array_equal(a[1], b[1]), "N=%d: out_norm differs" % N


# mix and norm -------------------------------------------------------------

def check_n0_textbook(orc):
    """N = 0: one source, weight 1, the mixture is the updated prefix: the
    call is plain add + RMSNorm (textbook RMSNorm in numpy)."""
    for eps in (1e-6, 0.25, 3.0):
        case = rand_case(5, 768, 0, add2=True, seed=20)
        out_prefix, out_norm, y, alpha = orc.fwd(case.prefix, case.add, case.add2, [],
                                                 case.query, case.gamma, eps,
                                                 want_f64=True, want_alpha=True)
        assert np.all(alpha == 1.0)
        p = torch_prefix(case.prefix, case.add, case.add2)
        assert np.array_equal(out_prefix, p)
        assert_close(y, textbook_rmsnorm(f64(p), case.gamma, eps), 1e-12, 1e-300, "N=0 eps=%g" % eps)


def check_self_snapshot_q0(orc):
    """N = 1 with the snapshot equal to the updated prefix and q = 0: the
    weights are exactly (1/2, 1/2) and the call reduces to add + RMSNorm."""
    case = rand_case(4, 1024, 0, add2=True, seed=21)
    p = torch_prefix(case.prefix, case.add, case.add2)
    q = np.zeros_like(case.query)
    _, _, y, alpha = orc.fwd(case.prefix, case.add, case.add2, [p], q, case.gamma,
                             case.eps, want_f64=True, want_alpha=True)
    assert np.all(alpha == 0.5), alpha
    assert_close(y, textbook_rmsnorm(f64(p), case.gamma, case.eps), 1e-12, 1e-300, "self snapshot")


def check_q0_uniform_mean(orc):
    """q = 0 makes every logit 0: weights 1/(N+1) and the mixture is the plain
    mean of the raw sources (of different magnitudes here)."""
    M, H, N = 3, 640, 6
    case = rand_case(M, H, N, add2=True, seed=22)
    snaps = [scale_pow2(s, k) for s, k in zip(case.snapshots, (-3, -1, 0, 1, 2, 4))]
    q = np.zeros_like(case.query)
    _, _, y, alpha = orc.fwd(case.prefix, case.add, case.add2, snaps, q, case.gamma,
                             case.eps, want_f64=True, want_alpha=True)
    assert_close(alpha, np.full((M, N + 1), 1.0 / (N + 1)), 1e-15, 0, "uniform alpha")
    p = torch_prefix(case.prefix, case.add, case.add2)
    mean = np.mean(np.stack([f64(s) for s in snaps] + [f64(p)]), axis=0)
    assert_close(y, textbook_rmsnorm(mean, case.gamma, case.eps), 1e-12, 1e-300, "q=0 mean")


def check_identical_sources(orc):
    """Every source equal to the updated prefix: whatever the weights, the
    mixture is that source."""
    case = rand_case(3, 512, 0, add2=True, seed=23)
    p = torch_prefix(case.prefix, case.add, case.add2)
    _, _, y = orc.fwd(case.prefix, case.add, case.add2, [p] * 7, case.query, case.gamma,
                      case.eps, want_f64=True)
    assert_close(y, textbook_rmsnorm(f64(p), case.gamma, case.eps), 1e-13, 1e-300, "identical")


def check_mix_output(orc):
    """The pre-norm mixture output (the capture tap of the "Model" section).
    N = 0 and identical sources: the mixture is the updated prefix, bit for
    bit.  q = 0: it is the plain numpy mean of the sources.  Always: the bf16
    mixture is the binary64 one rounded once, and out_norm is the textbook
    RMSNorm of that binary64 mixture."""
    case = rand_case(4, 768, 0, add2=True, seed=30)
    p = torch_prefix(case.prefix, case.add, case.add2)
    _, _, mix, mix64 = orc.fwd(case.prefix, case.add, case.add2, [], case.query, case.gamma,
                               case.eps, want_mix=True, want_mix_f64=True)
    assert np.array_equal(mix, p) and np.array_equal(mix64, f64(p)), "N=0 mixture"
    _, _, mix, mix64 = orc.fwd(case.prefix, case.add, case.add2, [p] * 5, case.query, case.gamma,
                               case.eps, want_mix=True, want_mix_f64=True)
    assert np.array_equal(mix, p), "identical sources mixture"
    assert_close(mix64, f64(p), 1e-15, 0, "identical sources mixture f64")

    M, H, N = 3, 640, 6
    case = rand_case(M, H, N, add2=True, seed=31)
    snaps = [scale_pow2(s, k) for s, k in zip(case.snapshots, (-3, -1, 0, 1, 2, 4))]
    q = np.zeros_like(case.query)
    _, _, mix, mix64 = orc.fwd(case.prefix, case.add, case.add2, snaps, q, case.gamma, case.eps,
                               want_mix=True, want_mix_f64=True)
    p = torch_prefix(case.prefix, case.add, case.add2)
    stack = np.stack([f64(s) for s in snaps] + [f64(p)])
    mean = np.mean(stack, axis=0)
    # binary64 summation error, bounded by the magnitudes of the terms
    assert_close(mix64, mean, 1e-12, 1e-15 * np.mean(np.abs(stack), axis=0), "q=0 mixture")
    rounded = np.array([orc.round_bf16(v) for v in mix64.ravel()], np.uint16).reshape(M, H)
    assert np.array_equal(mix, rounded), "mixture rounded once"

    case = rand_case(3, 896, 5, add2=True, seed=32)
    _, _, y, mix, mix64 = orc.fwd(case.prefix, case.add, case.add2, case.snapshots, case.query,
                                  case.gamma, case.eps, want_f64=True, want_mix=True,
                                  want_mix_f64=True)
    assert_close(y, textbook_rmsnorm(mix64, case.gamma, case.eps), 1e-12, 1e-300, "norm of mixture")
    rounded = np.array([orc.round_bf16(v) for v in mix64.ravel()], np.uint16).reshape(mix.shape)
    assert np.array_equal(mix, rounded), "mixture rounded once (random case)"


def check_dominant_logit(orc):
    """A query aligned with one RMS-normalised source gives it a logit of
    about 4H (~1000 here): its weight is exactly 1 in binary64 (the others
    underflow), no overflow happens, and the output is RMSNorm of that source."""
    M, H, N = 3, 256, 4
    case = rand_case(M, H, N, add2=True, seed=24)
    v = f64(case.snapshots[2][0])
    snap2 = np.repeat(case.snapshots[2][:1], M, axis=0)
    snaps = list(case.snapshots)
    snaps[2] = snap2
    q = W.to_bf16_bits(4.0 * v / np.sqrt(np.mean(v * v)))
    _, _, y, alpha = orc.fwd(case.prefix, case.add, case.add2, snaps, q, case.gamma,
                             case.eps, want_f64=True, want_alpha=True)
    assert np.all(np.isfinite(alpha))
    assert np.all(alpha[:, 2] == 1.0), alpha
    assert_close(y, textbook_rmsnorm(f64(snap2), case.gamma, case.eps), 1e-13, 1e-300, "dominant")


def check_two_source_closed_form(orc):
    """H = 8, eps = 0, one snapshot of ones (mean square 1) and an updated
    prefix [2,0,2,0,...] (mean square 2), q = (1/2, 0, ..., 0).  Logits
    1/2 and 1/sqrt(2); the prefix weight is the logistic
    a = 1/(1 + exp(1/2 - 1/sqrt(2))); the mixture is 1+a at even and 1-a at
    odd columns, its mean square 1 + a^2, so y = (1 +- a)/sqrt(1 + a^2) * gamma."""
    H = 8
    ones = np.full((1, H), 0x3F80, np.uint16)
    prefix = np.array([[0x4000, 0x0000] * 4], np.uint16)  # 2, 0, ...
    add = np.zeros((1, H), np.uint16)
    q = np.zeros(H, np.uint16)
    q[0] = 0x3F00  # 0.5
    gamma = np.array([0x3F80, 0x4000, 0x3F00, 0x3FC0, 0x3F80, 0x3F80, 0x4040, 0x3E80], np.uint16)
    _, _, y, alpha = orc.fwd(prefix, add, None, [ones], q, gamma, 0.0, want_f64=True, want_alpha=True)
    a = 1.0 / (1.0 + math.exp(0.5 - 1.0 / math.sqrt(2.0)))
    assert_close(alpha[0], [1.0 - a, a], 1e-15, 0, "closed-form alpha")
    x = np.array([1 + a, 1 - a] * 4)
    want = x / math.sqrt(1 + a * a) * f64(gamma)
    assert_close(y[0], want, 1e-14, 0, "closed-form y")


def check_two_source_eps_closed_form(orc):
    """The same two sources with eps = 1 and a gamma that is not 1 at the
    query's only nonzero column.  The key RMSNorm takes eps inside its square
    root: the snapshot of ones (mean square 1) gets the logit
    (1/2)/sqrt(1 + 1), the prefix [2,0,2,0,...] (mean square 2) gets
    1/sqrt(2 + 1); the query enters the logits as it is (gamma belongs to the
    final RMSNorm only).  The mixture is a0 + 2 a1 at even columns and a0 at
    odd ones (a1 the prefix weight, a0 = 1 - a1), its mean square
    ((a0 + 2 a1)^2 + a0^2)/2, and y = x / sqrt(that + 1) * gamma."""
    H = 8
    ones = np.full((1, H), 0x3F80, np.uint16)
    prefix = np.array([[0x4000, 0x0000] * 4], np.uint16)
    add = np.zeros((1, H), np.uint16)
    q = np.zeros(H, np.uint16)
    q[0] = 0x3F00  # 0.5
    gamma = np.array([0x4000, 0x3F00, 0x3FC0, 0x3E80, 0x3F80, 0x4040, 0x3F40, 0x3FA0], np.uint16)
    eps = 1.0
    _, _, y, alpha = orc.fwd(prefix, add, None, [ones], q, gamma, eps, want_f64=True, want_alpha=True)
    z0 = 0.5 / math.sqrt(1.0 + eps)
    z1 = 1.0 / math.sqrt(2.0 + eps)
    a1 = 1.0 / (1.0 + math.exp(z0 - z1))
    a0 = 1.0 - a1
    assert_close(alpha[0], [a0, a1], 1e-14, 0, "eps closed-form alpha")
    x = np.array([a0 + 2 * a1, a0] * 4)
    ms = ((a0 + 2 * a1) ** 2 + a0 ** 2) / 2
    want = x / math.sqrt(ms + eps) * f64(gamma)
    assert_close(y[0], want, 1e-14, 0, "eps closed-form y")


# exact evaluation at tiny H (rationals, then 60 significant digits) ---------

def _round_frac(x: Fraction, p: int, emin: int) -> Fraction:
    """x rounded to the nearest floating-point value with p significand bits
    (implicit bit included) and minimum normal exponent emin, ties to even,
    gradual underflow.  (No overflow: the tiny-H cases stay far from it.)"""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:  # bring a into [2^E, 2^(E+1))
        E -= 1
    E = max(E, emin)
    quantum = Fraction(2) ** (E - (p - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def _bf16_frac(bits) -> list:
    return [Fraction(float(v)) for v in W.bf16_bits_to_f32(np.asarray(bits, np.uint16)).ravel()]


def _frac_to_bf16_bits(v: Fraction) -> int:
    """A Fraction that is a bf16 value -> its bit pattern (exact)."""
    return int(W.to_bf16_bits(np.array([float(v)]))[0])


def exact_attnres(prefix, add, add2, snapshots, query, gamma, eps):
    """The operation on one token, evaluated from its definition without
    binary64: the fold-add in exact rationals rounded to binary32 and then to
    bf16 at each addition (round to nearest even, gradual underflow); the key
    RMSNorm, the logits, the softmax, the mixture and the final RMSNorm in
    exact rationals where they are rational and otherwise in 60-digit decimal
    arithmetic (square roots and exponentials correctly rounded at that
    precision).  Returns (out_prefix bits, y, alpha, x): y (the normalised
    output), alpha (the weights) and x (the pre-norm mixture) as lists of
    Decimal."""
    from decimal import Decimal, localcontext

    H = len(prefix)
    p, a = _bf16_frac(prefix), _bf16_frac(add)
    a2 = None if add2 is None else _bf16_frac(add2)
    q, g = _bf16_frac(query), _bf16_frac(gamma)
    e = Fraction(float(np.float32(eps)))
    f32 = lambda v: _round_frac(v, 24, -126)
    b16 = lambda v: _round_frac(v, 8, -126)
    pp = []
    for h in range(H):
        t = a[h] if a2 is None else b16(f32(a[h] + a2[h]))
        pp.append(b16(f32(p[h] + t)))
    sources = [_bf16_frac(s) for s in snapshots] + [pp]
    with localcontext() as ctx:
        ctx.prec = 60
        D = lambda fr: Decimal(fr.numerator) / Decimal(fr.denominator)
        z = []
        for k in sources:
            ms = sum(v * v for v in k) / H + e
            qk = sum(qh * v for qh, v in zip(q, k))
            z.append(D(qk) / D(ms).sqrt())
        zmax = max(z)
        ex = [(zs - zmax).exp() for zs in z]
        den = sum(ex)
        alpha = [w / den for w in ex]
        x = [sum(al * D(k[h]) for al, k in zip(alpha, sources)) for h in range(H)]
        msx = sum(v * v for v in x) / H + D(e)
        r = 1 / msx.sqrt()
        y = [x[h] * r * D(g[h]) for h in range(H)]
    return [_frac_to_bf16_bits(v) for v in pp], y, alpha, x


def _tiny_h_cases(seed=41):
    """Seeded one-token calls at H = 8, 16, 64: eps from 0 to 3, sources of
    mean square 1e-4 .. 10 (so eps moves every logit and the final scale),
    a query of logits O(1) on every column, gamma far from 1, with and without
    the second addend, N from 0 to 12."""
    rng = np.random.default_rng(seed)
    out = []
    for H in (8, 16, 64):
        for N, eps, add2 in ((0, 0.25, True), (1, 1e-3, False), (3, 0.25, True), (6, 3.0, True),
                             (12, 1e-3, True), (4, 0.0, False), (2, 3.0, False)):
            scale = lambda: 10.0 ** rng.uniform(-2.0, 0.5)
            bf = lambda x: W.to_bf16_bits(np.asarray(x, np.float64))
            s_p = scale()
            prefix = bf(s_p * rng.standard_normal(H))
            add = bf(0.5 * s_p * rng.standard_normal(H))
            add2v = bf(0.5 * s_p * rng.standard_normal(H)) if add2 else None
            snaps = [bf(scale() * rng.standard_normal(H)) for _ in range(N)]
            query = bf(rng.standard_normal(H) * 2.0 / math.sqrt(H))
            gamma = bf(1.0 + 0.4 * rng.standard_normal(H))
            out.append((H, N, eps, prefix, add, add2v, snaps, query, gamma))
    return out


def check_exact_tiny_h(orc):
    """The oracle's binary64 result against an exact evaluation of the same
    definition (exact_attnres) on one-token calls at H = 8, 16 and 64:
    out_prefix bit for bit, the weights and the unrounded out_norm to 1e-12
    of the row's largest value (binary64 leaves about 1e-15; a changed term of
    the key RMSNorm, the logits, the softmax or the final RMSNorm moves them
    by far more), the same for the pre-norm mixture, and the bits of out_norm
    and of the mixture output equal to the exact values rounded to nearest
    even wherever those are not within 1e-12 of a tie."""
    for H, N, eps, prefix, add, add2v, snaps, query, gamma in _tiny_h_cases():
        what = "H=%d N=%d eps=%g" % (H, N, eps)
        row = lambda v: None if v is None else v.reshape(1, H)
        op, on, y, alpha, mix, mix64 = orc.fwd(row(prefix), row(add), row(add2v), [row(s) for s in snaps], query,
                                               gamma, eps, want_f64=True, want_alpha=True, want_mix=True,
                                               want_mix_f64=True)
        xp, xy, xa, xx = exact_attnres(prefix, add, add2v, snaps, query, gamma, eps)
        assert np.array_equal(op[0], np.array(xp, np.uint16)), what + ": out_prefix"
        xa = np.array([float(v) for v in xa])
        assert_close(alpha[0], xa, 0, 1e-12, what + ": alpha")
        for name, got64, got16, exact in (("out_norm", y, on, xy), ("mixture", mix64, mix, xx)):
            ex = np.array([float(v) for v in exact])
            scale = np.max(np.abs(ex))
            assert scale > 0.05 or name == "mixture", what + ": degenerate case"
            assert_close(got64[0], ex, 0, 1e-12 * scale, "%s: %s before rounding" % (what, name))
            for h in range(H):
                want = _nearest_bf16_fraction(ex[h])
                lo = _nearest_bf16_fraction(ex[h] * (1 - 1e-12))
                hi = _nearest_bf16_fraction(ex[h] * (1 + 1e-12))
                if lo == hi == want:
                    assert got16[0, h] == want, "%s: %s[%d] %04x, exact rounds to %04x" % (
                        what, name, h, got16[0, h], want)


def check_token_permutation(orc):
    """Tokens are independent: permuting the rows of every [M,H] input
    permutes the outputs, bit for bit."""
    case = rand_case(6, 512, 3, add2=True, seed=25)
    perm = np.array([3, 0, 5, 1, 4, 2])
    a = orc.fwd(case.prefix, case.add, case.add2, case.snapshots, case.query, case.gamma, case.eps)
    c = case.rows(perm)
    b = orc.fwd(c.prefix, c.add, c.add2, c.snapshots, c.query, c.gamma, c.eps)
    assert np.array_equal(a[0][perm], b[0]) and np.array_equal(a[1][perm], b[1])


def check_snapshot_scale_invariance(orc):
    """eps = 0: scaling one snapshot by 2^k leaves every logit, hence every
    weight, unchanged bit for bit (the key RMSNorm removes the scale);
    scaling all inputs by 2^k scales the updated prefix by 2^k and leaves the
    unrounded output unchanged bit for bit."""
    case = rand_case(3, 512, 4, add2=True, seed=26)
    base = orc.fwd(case.prefix, case.add, case.add2, case.snapshots, case.query, case.gamma,
                   0.0, want_f64=True, want_alpha=True)
    for j, k in ((0, 3), (2, -5), (3, 7)):
        snaps = list(case.snapshots)
        snaps[j] = scale_pow2(snaps[j], k)
        r = orc.fwd(case.prefix, case.add, case.add2, snaps, case.query, case.gamma, 0.0,
                    want_alpha=True)
        assert np.array_equal(r[2], base[3]), "weights changed when scaling snapshot %d" % j
    k = 4
    s = lambda b: scale_pow2(b, k)
    r = orc.fwd(s(case.prefix), s(case.add), s(case.add2), [s(x) for x in case.snapshots],
                case.query, case.gamma, 0.0, want_f64=True, want_alpha=True)
    assert np.array_equal(r[0], s(base[0])), "updated prefix does not scale"
    assert np.array_equal(r[3], base[3]), "weights changed under global scaling"
    assert np.array_equal(r[2], base[2]), "output changed under global scaling"


def check_snapshot_permutation(orc):
    """Reordering the snapshots permutes the weights and changes the output
    only by summation-order rounding."""
    case = rand_case(3, 512, 5, add2=True, seed=27)
    a = orc.fwd(case.prefix, case.add, case.add2, case.snapshots, case.query, case.gamma,
                case.eps, want_f64=True, want_alpha=True)
    perm = [4, 2, 0, 3, 1]
    b = orc.fwd(case.prefix, case.add, case.add2, [case.snapshots[i] for i in perm],
                case.query, case.gamma, case.eps, want_f64=True, want_alpha=True)
    assert_close(b[3][:, :5], a[3][:, perm], 1e-13, 1e-300, "permuted alpha")
    assert_close(b[2], a[2], 1e-12, 1e-300, "permuted output")


def check_round_vs_fractions(orc, n=20000, seed=5):
    """oracle_round_bf16 on binary64 inputs (including constructed near-ties
    and the subnormal range) against the nearest bf16 found with exact
    rational arithmetic."""
    rng = np.random.default_rng(seed)
    xs = list(rng.standard_normal(n // 4) * np.exp2(rng.integers(-140, 128, n // 4)))
    # ties and near-ties: midpoints between adjacent bf16 values, nudged
    for _ in range(n // 4):
        e = int(rng.integers(-133, 120))
        m = int(rng.integers(0, 256))
        mid = (2 * m + 1) * 2.0 ** (e - 1)
        for d in (0.0, 1e-12, -1e-12):
            xs.append(float(mid * (1 + d)) * (1 if rng.random() < 0.5 else -1))
    for x in xs:
        got = orc.round_bf16(x)
        want = _nearest_bf16_fraction(x)
        assert got == want, "round(%r): got %04x want %04x" % (x, got, want)


_BF16_POS = None


def _bf16_table():
    global _BF16_POS
    if _BF16_POS is None:
        vals = []
        for b in range(0x7F80 + 1):  # 0 .. +Inf
            vals.append(Fraction(float(W.bf16_bits_to_f32(np.array([b], np.uint16))[0])) if b < 0x7F80 else None)
        _BF16_POS = vals
    return _BF16_POS


def _nearest_bf16_fraction(x: float) -> int:
    import bisect

    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = Fraction(abs(x))
    tab = _bf16_table()
    finite = tab[:0x7F80]
    i = bisect.bisect_left(finite, a)
    if i < len(finite) and finite[i] == a:
        return sign | i
    if i == len(finite):  # beyond max
        lo, hi = 0x7F7F, None
    else:
        lo, hi = i - 1, i
    top = Fraction(2) ** 128  # the value "one ulp past max" for the tie rule
    hv = finite[hi] if hi is not None else top
    lv = finite[lo]
    dl, dh = a - lv, hv - a
    if dl < dh:
        r = lo
    elif dh < dl:
        r = hi if hi is not None else 0x7F80
    else:
        r = lo if lo % 2 == 0 else (hi if hi is not None else 0x7F80)
    return sign | r


# registry ----------------------------------------------------------------

QUICK = [
    check_golden_fold,
    check_prefix_vs_torch,
    check_add2_equals_presummed,
    check_n0_textbook,
    check_self_snapshot_q0,
    check_q0_uniform_mean,
    check_identical_sources,
    check_mix_output,
    check_two_source_closed_form,
    check_two_source_eps_closed_form,
    check_exact_tiny_h,
    check_dominant_logit,
    check_token_permutation,
    check_snapshot_scale_invariance,
    check_snapshot_permutation,
]
