"""GPU: the 25-layer decoder chain at its full size (256 tokens, H = 7168).

Page "[#20545][perf] Kimi K3: fold the MoE-tail additions into the next
attention-residual", section "Test Coverage": the chain with MoE tails deferred
into the next fused call equals the eager chain bit for bit, snapshot bank
included.  Here the eager chain adds routed + shared with the standalone add
kernel and calls the fused op with one addend; the deferred chain folds both.
Every layer is also checked against the oracle chain on sampled token rows
(tokens are independent, so the oracle runs only those rows).
"""
import numpy as np
import pytest

import parity as P
from attention_residual_rmsnorm_amd import workloads as W

pytestmark = pytest.mark.gpu


def gpu_chain(ar, chain, deferred: bool):
    import torch

    d = P.dev
    dev_layers = [(d(l.query), d(l.gamma), d(l.routed), d(l.shared)) for l in chain.layers]

    def step(l, prefix, bank, layer):
        q, g, r, s = dev_layers[l]
        if deferred:
            return ar.attnres_add_rmsnorm_fwd(prefix, r, s, bank, q, g, chain.eps)
        t = ar.attnres_bf16_add(r, s)
        return ar.attnres_add_rmsnorm_fwd(prefix, t, None, bank, q, g, chain.eps)

    zero = lambda: torch.zeros((chain.M, chain.H), dtype=torch.bfloat16, device="cuda")
    outs, bank = W.run_chain(chain, step, zero, embedding=d(chain.embedding), prefix0=d(chain.prefix0))
    torch.cuda.synchronize()
    return [(P.host(a), P.host(b)) for a, b in outs], [P.host(b) for b in bank]


@pytest.fixture(scope="module")
def chain():
    return W.make_chain()


@pytest.fixture(scope="module")
def ar():
    import attention_residual_rmsnorm_amd as ar

    ar.attnres_init()
    yield ar
    ar.attnres_set_variant(0, 0)


@pytest.mark.parametrize("variant", [(0, 0), (2, 0)], ids=["auto", "S"])
def test_chain_deferred_equals_eager_and_oracle(ar, orc, chain, variant):
    ar.attnres_set_variant(*variant)
    try:
        print("chain variant", variant, ar.attnres_plan(chain.M, 12, chain.H), flush=True)
        out_d, bank_d = gpu_chain(ar, chain, deferred=True)
        out_e, bank_e = gpu_chain(ar, chain, deferred=False)
    finally:
        ar.attnres_set_variant(0, 0)
    assert len(bank_d) == len(bank_e) == 12
    for l, ((pd, nd), (pe, ne)) in enumerate(zip(out_d, out_e)):
        assert np.array_equal(pd, pe), "layer %d out_prefix deferred != eager" % l
        assert np.array_equal(nd, ne), "layer %d out_norm deferred != eager" % l
    for a, b in zip(bank_d, bank_e):
        assert np.array_equal(a, b)

    idx = np.unique(np.r_[0, 1, 127, 254, 255, np.random.default_rng(1).integers(0, chain.M, 11)])
    sub = chain.rows(idx)
    zero = lambda: np.zeros((sub.M, sub.H), np.uint16)
    step = lambda l, p, b, L: orc.fwd(p, L.routed, L.shared, b, L.query, L.gamma, sub.eps)
    ref, _ = W.run_chain(sub, step, zero)
    for l, ((gp, gn), (rp, rn)) in enumerate(zip(out_d, ref)):
        P.assert_parity(gp[idx], gn[idx], rp, rn, "chain layer %d" % l)
    assert ar.attnres_debug_timeouts() == 0
