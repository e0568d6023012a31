"""CPU test of the 25-layer decoder chain hand-off, on the oracle.

Page "[#20545][perf] Kimi K3: fold the MoE-tail additions into the next
attention-residual", section "Test Coverage": a 25-layer chain whose MoE tails
are deferred into the next fused call is bitwise equal to the eager chain,
snapshot bank included; section "Model": the updated prefix written to the
bank or carried on is bitwise the same as without the fold.

Deferred: each call receives (routed, shared) as its two addends.
Eager:    PyTorch adds routed + shared first (bf16 tensor add), the call
          receives the single sum.  Every layer's updated prefix must also
          equal PyTorch's prefix + (routed + shared).
"""
import numpy as np

import pins
from attention_residual_rmsnorm_amd import workloads as W


def test_chain_schedule():
    sched = W.chain_schedule()
    assert len(sched) == 25
    assert [n for n, _ in sched][:6] == [1, 1, 2, 2, 3, 3]
    assert sched[-1] == (12, False) and max(n for n, _ in sched) == 12
    assert sum(n for n, _ in sched) == 168
    assert sum(p for _, p in sched) == 11


def test_chain_deferred_equals_eager(orc):
    chain = W.make_chain(M=6, H=1024)
    zero = lambda: np.zeros((chain.M, chain.H), np.uint16)

    def deferred(l, prefix, bank, layer):
        return orc.fwd(prefix, layer.routed, layer.shared, bank, layer.query, layer.gamma, chain.eps)

    def eager(l, prefix, bank, layer):
        t = pins.bits_of(pins.tbf(layer.routed) + pins.tbf(layer.shared))
        out = orc.fwd(prefix, t, None, bank, layer.query, layer.gamma, chain.eps)
        want = pins.bits_of(pins.tbf(prefix) + pins.tbf(t))
        assert np.array_equal(out[0], want), "layer %d prefix != torch" % l
        return out

    out_d, bank_d = W.run_chain(chain, deferred, zero)
    out_e, bank_e = W.run_chain(chain, eager, zero)
    assert len(bank_d) == len(bank_e) == 12
    for l, ((pd, nd), (pe, ne)) in enumerate(zip(out_d, out_e)):
        assert np.array_equal(pd, pe), "layer %d out_prefix" % l
        assert np.array_equal(nd, ne), "layer %d out_norm" % l
    for a, b in zip(bank_d, bank_e):
        assert np.array_equal(a, b)


def test_chain_rows_independent(orc):
    """Running the chain on a subset of tokens reproduces those rows of the
    full chain (what lets the full-size GPU chain be checked on sampled rows)."""
    chain = W.make_chain(M=5, H=512)
    zero_full = lambda: np.zeros((chain.M, chain.H), np.uint16)
    step = lambda l, p, b, L, c=chain: orc.fwd(p, L.routed, L.shared, b, L.query, L.gamma, c.eps)
    full, _ = W.run_chain(chain, step, zero_full)
    idx = [4, 1]
    sub = chain.rows(idx)
    part, _ = W.run_chain(sub, lambda l, p, b, L: orc.fwd(p, L.routed, L.shared, b, L.query, L.gamma, sub.eps),
                          lambda: np.zeros((sub.M, sub.H), np.uint16))
    for (pf, nf), (ps, ns) in zip(full, part):
        assert np.array_equal(pf[idx], ps) and np.array_equal(nf[idx], ns)
