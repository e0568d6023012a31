"""GPU parity of the pre-norm mixture output (attnres_add_rmsnorm_mix_fwd).

The page "[#20545][perf] Kimi K3: fold the MoE-tail additions into the next
attention-residual", section "Model", keeps a layer with a speculative-decoding
hidden-state capture off the fused path because the tap needs the pre-norm
mixture; the mix entry point writes it in the same launch.  Checked here:
out_mix against the oracle's mixture (out_norm's bar), out_prefix / out_norm
bitwise equal to the plain call's, N = 0 (mixture = updated prefix, exactly),
ragged shapes, canaries, and a NULL out_mix through the C ABI.
"""
import ctypes
import sys

import numpy as np
import pytest

import parity as P
from attention_residual_rmsnorm_amd import workloads as W

pytestmark = pytest.mark.gpu

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


@pytest.mark.parametrize("variant", VARIANTS, ids=VID, indirect=True)
@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_mix_named_workload(ar, orc, variant, name):
    case = W.config_case(name)
    if not supported(ar, case.M, case.N, case.H):
        pytest.skip("variant not available for this size")
    say("mix case", name, "variant", variant, ar.attnres_plan(case.M, case.N, case.H))
    gp, gn, gm = P.run_gpu_mix(case)
    rp, rn, rm = P.run_oracle_mix(orc, case)
    P.assert_parity(gp, gn, rp, rn, name)
    P.assert_mix_parity(gm, rm, name)
    pp, pn = P.run_gpu(case)
    assert np.array_equal(pp, gp) and np.array_equal(pn, gn), "mix call changed out_prefix/out_norm"


@pytest.mark.parametrize("variant", VARIANTS, ids=VID, indirect=True)
@pytest.mark.parametrize("M,H,N", [(1, 8, 0), (3, 8, 12), (5, 520, 3), (3, 1000, 12), (4, 4104, 7),
                                   (2, 7176, 12), (33, 7168, 9), (3, 16384, 12)])
def test_mix_shapes(ar, orc, variant, M, H, N):
    if not supported(ar, M, N, H):
        pytest.skip("variant not available for this size")
    case = W.make_case(cfg=80, M=M, H=H, N=N, add2=(N % 2 == 0))
    say("mix shape", M, H, N, "variant", variant, ar.attnres_plan(M, N, H))
    gp, gn, gm = P.run_gpu_mix(case)
    rp, rn, rm = P.run_oracle_mix(orc, case)
    P.assert_parity(gp, gn, rp, rn, "M=%d H=%d N=%d" % (M, H, N))
    P.assert_mix_parity(gm, rm, "M=%d H=%d N=%d" % (M, H, N))


@pytest.mark.parametrize("variant", [(1, 0), (2, 0)], ids=["W", "S"], indirect=True)
def test_mix_without_snapshots_is_the_prefix(ar, variant):
    """N = 0: one source with weight 1, so the mixture is p' bit for bit."""
    case = W.make_case(cfg=81, M=6, N=0, add2=True)
    gp, _, gm = P.run_gpu_mix(case)
    assert np.array_equal(gm, gp)


@pytest.mark.parametrize("variant", [(1, 0), (2, 0)], ids=["W", "S"], indirect=True)
def test_mix_canaries(ar, orc, variant):
    import torch

    case = W.make_case(cfg=82, M=5, H=1000, N=4, add2=True)
    n = case.M * case.H
    pad = 4096
    canary = 0x7E57
    buf = torch.full((n + 2 * pad,), canary, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    outm = buf[pad:pad + n].view(case.M, case.H)
    d = P.dev
    ar.attnres_add_rmsnorm_mix_fwd(d(case.prefix), d(case.add), d(case.add2), [d(s) for s in case.snapshots],
                                   d(case.query), d(case.gamma), case.eps, out_mix=outm)
    h = P.host(buf)
    assert np.all(h[:pad] == canary) and np.all(h[pad + n:] == canary)
    P.assert_mix_parity(P.host(outm), P.run_oracle_mix(orc, case)[2], "canary")


def test_mix_null_is_the_plain_call(ar):
    """A NULL out_mix through the C ABI gives the plain call's bits."""
    import torch

    case = W.make_case(cfg=83, M=8, N=6, add2=True)
    d = P.dev
    ins = [d(case.prefix), d(case.add), d(case.add2)] + [d(s) for s in case.snapshots] + [d(case.query),
                                                                                          d(case.gamma)]
    op, on = torch.empty_like(ins[0]), torch.empty_like(ins[0])
    vp = ctypes.c_void_p
    arr = (vp * case.N)(*[t.data_ptr() for t in ins[3:3 + case.N]])
    rc = ar.library().attnres_add_rmsnorm_mix_fwd(
        ins[0].data_ptr(), ins[1].data_ptr(), ins[2].data_ptr(), arr, case.N, ins[-2].data_ptr(),
        ins[-1].data_ptr(), ctypes.c_float(case.eps), case.M, case.H, op.data_ptr(), on.data_ptr(), None,
        torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    pp, pn = P.run_gpu(case)
    assert np.array_equal(P.host(op), pp) and np.array_equal(P.host(on), pn)


@pytest.mark.parametrize("variant", [(1, 0), (2, 0)], ids=["W", "S"], indirect=True)
def test_mix_graph_replay(ar, variant):
    """The mixture call captured into a HIP graph and replayed with fresh inputs:
    every replay equals the eager call, bit for bit."""
    import torch

    cases = [W.make_case(cfg=84 + i, M=16, N=7, add2=True) for i in range(3)]
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
    assert ar.attnres_debug_timeouts() == 0
