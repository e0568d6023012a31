"""GPU parity beyond one pass of sources: 13..64 snapshots.

The page "[#20545][perf] Kimi K3: fold the MoE-tail additions into the next
attention-residual", section "Model", sends calls with more than 12 snapshot
sources down an unfused fallback.  Here kernel W takes them in batches of 12
with the running softmax carried across batches.  Checked against the oracle
(out_prefix bit-exact, out_norm and the mixture within 2 bf16 ulps or 1e-2)
across batch boundaries (13, 24, 25, 36, 64 sources), ragged H, one and many
tokens, both vector widths, with and without the second addend.
"""
import sys

import numpy as np
import pytest

import parity as P
from attention_residual_rmsnorm_amd import workloads as W

pytestmark = pytest.mark.gpu


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


SHAPES = [(1, 7168, 13), (3, 7168, 24), (2, 7168, 25), (5, 1000, 36), (2, 520, 64), (33, 7168, 30),
          (2, 7176, 14), (3, 16384, 20), (1, 8, 64), (260, 512, 13), (1, 7168, 31), (17, 1000, 16), (8, 520, 31),
          # the split's two-wave form (32..63 snapshots: wave 1 holding 1 to 32 sources)
          (1, 7168, 32), (2, 7168, 33), (3, 7168, 47), (4, 7168, 48), (1, 7168, 63), (9, 8192, 50),
          (17, 896, 40), (12, 1000, 49), (1, 8, 63)]


@pytest.mark.parametrize("variant", [(0, 0), (1, 2), (1, 4), (2, 1), (2, 2)], ids=["auto", "W2", "W4", "S1w", "S2w"],
                         indirect=True)
@pytest.mark.parametrize("M,H,N", SHAPES)
def test_many_sources(ar, orc, variant, M, H, N):
    try:
        ar.attnres_plan(M, N, H)
    except ar.AttnResError:
        pytest.skip("variant not available for this size")
    case = W.make_case(cfg=85, M=M, H=H, N=N, add2=(N % 2 == 1))
    say("many sources", M, H, N, "variant", variant, ar.attnres_plan(M, N, H))
    gp, gn, gm = P.run_gpu_mix(case)
    rp, rn, rm = P.run_oracle_mix(orc, case)
    P.assert_parity(gp, gn, rp, rn, "M=%d H=%d N=%d" % (M, H, N))
    P.assert_mix_parity(gm, rm, "M=%d H=%d N=%d" % (M, H, N))


@pytest.mark.parametrize("H", [7168, 3584, 896, 16384])
@pytest.mark.parametrize("N", [13, 31])
@pytest.mark.parametrize("M", [16, 17, 32, 33, 64, 65, 96, 97])
def test_many_sources_dispatch_bounds(ar, orc, M, N, H):
    """The automatic dispatch above 12 snapshots on both sides of each token
    bound (at H = 7168 1-wave split chunks up to 16 tokens and from 33 to 64,
    2-wave from 17 to 32 and 65 to 96; shorter rows 1-wave up to 96; rows
    longer than 8192 1-wave from 17 to 32, else 2-wave; then kernel W's
    batches)."""
    case = W.make_case(cfg=86, M=M, H=H, N=N, add2=(M % 2 == 1))
    say("many sources, auto", M, H, N, ar.attnres_plan(M, N, case.H))
    gp, gn = P.run_gpu(case)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(gp, gn, rp, rn, "M=%d H=%d N=%d" % (M, H, N))


@pytest.mark.parametrize("H", [7168, 8192, 896, 16384])
@pytest.mark.parametrize("N", [32, 39, 40, 63])
@pytest.mark.parametrize("M", [1, 16, 17, 64, 65, 96, 97])
def test_split_long_dispatch_bounds(ar, orc, M, N, H):
    """The automatic dispatch from 32 to 63 snapshots on both sides of its
    bounds (rows of 7168 and more: the split kernel's two-wave form up to 16
    tokens where rows are at most 8192, its four-wave form beyond, up to 64
    tokens below 40 snapshots and 96 from 40 on; shorter rows the two-wave
    form up to 96; then kernel W's batches), with the pre-norm mixture
    output."""
    case = W.make_case(cfg=87, M=M, H=H, N=N, add2=(M % 2 == 0))
    say("two-wave split, auto", M, H, N, ar.attnres_plan(M, N, case.H))
    gp, gn, gm = P.run_gpu_mix(case)
    rp, rn, rm = P.run_oracle_mix(orc, case)
    P.assert_parity(gp, gn, rp, rn, "M=%d H=%d N=%d" % (M, H, N))
    P.assert_mix_parity(gm, rm, "M=%d H=%d N=%d" % (M, H, N))


def test_split_long_no_timeouts(ar):
    assert ar.attnres_debug_timeouts() == 0


def test_many_sources_scaled_and_presummed(ar, orc):
    """Sources of very different magnitudes across batches (the scaled
    workload's structure), and add2 == one pre-summed addend bitwise."""
    import dataclasses

    import pins

    case = W.make_case(cfg=86, M=4, N=40, add2=True, special="scaled")
    gp, gn = P.run_gpu(case)
    rp, rn = P.run_oracle(orc, case)
    P.assert_parity(gp, gn, rp, rn, "scaled N=40")
    t = pins.bits_of(pins.tbf(case.add) + pins.tbf(case.add2))
    b = P.run_gpu(dataclasses.replace(case, add=t, add2=None))
    assert np.array_equal(gp, b[0]) and np.array_equal(gn, b[1])


def test_many_sources_deterministic(ar):
    case = W.make_case(cfg=87, M=16, N=30, add2=True)
    first = P.run_gpu(case)
    for _ in range(5):
        again = P.run_gpu(case)
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])


def test_many_sources_graph_replay(ar):
    """A captured call with 20 sources and the mixture output, replayed with
    fresh inputs copied in between: every replay equals the eager call."""
    import torch

    cases = [W.make_case(cfg=88 + i, M=12, N=20, add2=True) for i in range(3)]
    c0 = cases[0]
    d = P.dev
    ins = dict(prefix=d(c0.prefix), add=d(c0.add), add2=d(c0.add2), snaps=[d(s) for s in c0.snapshots],
               query=d(c0.query), gamma=d(c0.gamma))
    outp, outn, outm = (torch.empty_like(ins["prefix"]) for _ in range(3))

    def call():
        ar.attnres_add_rmsnorm_mix_fwd(ins["prefix"], ins["add"], ins["add2"], ins["snaps"], ins["query"],
                                       ins["gamma"], c0.eps, out_prefix=outp, out_norm=outn, out_mix=outm)

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
    for rep in range(6):
        c = cases[rep % len(cases)]
        for key, src in (("prefix", c.prefix), ("add", c.add), ("add2", c.add2), ("query", c.query),
                         ("gamma", c.gamma)):
            ins[key].copy_(d(src))
        for t, src in zip(ins["snaps"], c.snapshots):
            t.copy_(d(src))
        for o in (outp, outn, outm):
            o.zero_()
        g.replay()
        torch.cuda.synchronize()
        ep, en, em = P.run_gpu_mix(c)
        assert np.array_equal(P.host(outp), ep) and np.array_equal(P.host(outn), en) \
            and np.array_equal(P.host(outm), em), "replay %d" % rep
