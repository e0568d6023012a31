"""attnres_add_rmsnorm_fwd_noalloc: the fused call for callers that cannot
allocate, through the C ABI, against attnres_add_rmsnorm_fwd.

Its split-kernel scratch is a static device array (96 token slots) instead of
the allocated one, so it needs no attnres_init.  The first test calls it before
anything in the process has called attnres_init (when the file runs alone),
two calls in a row with the second smaller, and then compares with the
allocating entry point (same kernels: the same bits) and with the oracle.
"""
import ctypes
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
    yield ar
    ar.attnres_set_variant(0, 0)


def noalloc_c(ar, case, out_prefix, out_norm):
    """One call of the no-allocation entry point through ctypes on the C ABI."""
    import torch

    d = lambda x: None if x is None else P.dev(x)
    ins = [d(case.prefix), d(case.add), d(case.add2), [d(s) for s in case.snapshots], d(case.query),
           d(case.gamma)]
    vp = ctypes.c_void_p
    ptr = lambda t: None if t is None else t.data_ptr()
    n = case.N
    arr = (vp * max(n, 1))(*[s.data_ptr() for s in ins[3]])
    rc = ar.library().attnres_add_rmsnorm_fwd_noalloc(
        ptr(ins[0]), ptr(ins[1]), ptr(ins[2]), arr if n else None, n, ptr(ins[4]), ptr(ins[5]),
        ctypes.c_float(case.eps), case.M, case.H, out_prefix.data_ptr(), out_norm.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return rc


def out_pair(M, H):
    import torch

    return (torch.empty((M, H), dtype=torch.bfloat16, device="cuda"),
            torch.empty((M, H), dtype=torch.bfloat16, device="cuda"))


# (M, N): the split kernel at the most tokens the automatic dispatch gives it
# (2-wave chunks, two exchanges), then smaller calls (1-wave chunks, two
# exchanges and the Gram form's one), one token, the most sources the split kernel
# takes, calls kernel W serves (no scratch), the hybrid of W and split chunks
# just past the CU count (its split part at the most tokens the automatic
# dispatch gives it), 2-wave chunks again, more than 12 snapshots at the
# most tokens the split takes them, and the split's two-wave form (32..63
# snapshots, its second record page) at its most tokens and at two, and the
# hybrid's half-row chunks at its most tokens
CALLS = [(96, 12), (48, 12), (8, 4), (1, 12), (64, 31), (256, 12), (3, 0), (320, 12), (300, 4), (92, 8), (96, 20),
         (96, 63), (2, 33), (352, 8)]


def test_noalloc_matches_fwd(ar, orc):
    cases = [W.make_case(cfg=85, M=M, N=N, add2=(i % 2 == 0)) for i, (M, N) in enumerate(CALLS)]
    got = []
    for case in cases:  # the no-allocation calls first, back to back
        say("noalloc call", case.M, case.N, ar.attnres_plan(case.M, case.N, case.H))
        op, on = out_pair(case.M, case.H)
        rc = noalloc_c(ar, case, op, on)
        assert rc == ar.ATTNRES_OK, ar.attnres_status_string(rc)
        got.append((P.host(op), P.host(on)))
    for case, (gp, gn) in zip(cases, got):
        ep, en = P.run_gpu(case)  # the allocating entry point (the binding runs attnres_init)
        assert np.array_equal(gp, ep), "M=%d N=%d: out_prefix differs from attnres_add_rmsnorm_fwd" % (case.M,
                                                                                                         case.N)
        P.assert_parity(gp, gn, ep, en, "noalloc vs fwd M=%d N=%d" % (case.M, case.N))
        assert np.array_equal(gn, en), "M=%d N=%d: same kernels, different bits" % (case.M, case.N)
        rp, rn = P.run_oracle(orc, case)
        P.assert_parity(gp, gn, rp, rn, "noalloc vs oracle M=%d N=%d" % (case.M, case.N))
    assert ar.attnres_debug_timeouts() == 0


def test_noalloc_rejects_beyond_static_scratch(ar):
    """The split kernel forced on 97 tokens: the allocating entry point serves
    it (512 slots), the no-allocation one (96 slots) returns ATTNRES_ESCRATCH;
    96 tokens it serves."""
    assert ar.ATTNRES_NOALLOC_MAX_SPLIT_TOKENS == 96
    case = W.make_case(cfg=86, M=97, N=8, add2=True)
    ar.attnres_set_variant(2, 2)
    try:
        op, on = out_pair(case.M, case.H)
        assert noalloc_c(ar, case, op, on) == ar.ATTNRES_ESCRATCH
        assert "static scratch" in ar.attnres_status_string(ar.ATTNRES_ESCRATCH)
        P.run_gpu(case)
    finally:
        ar.attnres_set_variant(0, 0)
    case = W.make_case(cfg=86, M=96, N=8, add2=True)
    ar.attnres_set_variant(2, 2)
    try:
        op, on = out_pair(case.M, case.H)
        assert noalloc_c(ar, case, op, on) == ar.ATTNRES_OK
        ep, en = P.run_gpu(case)
    finally:
        ar.attnres_set_variant(0, 0)
    assert np.array_equal(P.host(op), ep) and np.array_equal(P.host(on), en)


@pytest.mark.parametrize("N", [8, 4])  # two exchanges; the Gram form's one
def test_noalloc_graph_replay(ar, N):
    """The no-allocation call captured into a HIP graph and replayed with fresh
    inputs copied in between (eager work and synchronisation between
    replays): every replay equals the allocating entry point's eager call."""
    import torch

    cases = [W.make_case(cfg=87 + i, M=16, N=N, add2=True) for i in range(3)]
    c0 = cases[0]
    d = P.dev
    ins = dict(prefix=d(c0.prefix), add=d(c0.add), add2=d(c0.add2), snaps=[d(s) for s in c0.snapshots],
               query=d(c0.query), gamma=d(c0.gamma))
    outp, outn = out_pair(c0.M, c0.H)

    def call():
        ar.attnres_add_rmsnorm_fwd_noalloc(ins["prefix"], ins["add"], ins["add2"], ins["snaps"], ins["query"],
                                           ins["gamma"], c0.eps, outp, outn)

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
    for rep in range(9):
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
        ep, en = P.run_gpu(c)
        assert np.array_equal(P.host(outp), ep) and np.array_equal(P.host(outn), en), "replay %d" % rep
