"""Seeded synthetic workloads for the fused AttnRes + RMSNorm decode step.

This module only draws inputs: it holds none of the operation's arithmetic.
Both the parity tests (against the CPU oracle) and the benchmark take their
inputs from here; every tensor is returned as a numpy array of bf16 bit
patterns (``uint16``).

Shapes follow the decode shapes on the page "[#20545][perf] Kimi K3: fold the
MoE-tail additions into the next attention-residual" (section "Model": hidden
size 7168, BF16, a fused window of up to 32 tokens per rank, at most 12
snapshot-bank sources), plus a 256-token bandwidth case.

Recipe (also stated in the design notes):
  * each tensor is drawn in float64 from ``numpy.random.Generator(PCG64)``
    seeded by (workload id, tensor name[, layer]) and rounded to bf16
    (round-to-nearest-even via torch's CPU conversion float32 -> bfloat16);
  * N(mu, sigma) means standard deviation sigma;
  * query ~ N(0, 1/sqrt(H)), gamma = 1 + N(0, 0.1), eps = 1e-6;
  * prefix, add and snapshots ~ N(0, 1); routed and shared (add, add2 of the
    MoE tail) ~ N(0, 0.5).
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import Dict, List, Optional, Sequence

import numpy as np

H_MODEL = 7168
EPS = 1e-6
MAX_SOURCES = 12  # snapshot-bank sources the fused window accepts


def _rng(*key) -> np.random.Generator:
    words = []
    for k in key:
        if isinstance(k, str):
            words.append(zlib.crc32(k.encode()))
        else:
            words.append(int(k))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(words)))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (numpy RNE) -> bfloat16 bits (torch RNE)."""
    import torch

    f32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (for building inputs and reports)."""
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def normal(key, shape, sigma=1.0, mu=0.0) -> np.ndarray:
    return to_bf16_bits(mu + sigma * _rng(*key).standard_normal(shape))


@dataclasses.dataclass
class Case:
    """One call's inputs (bf16 bits) and its description."""

    name: str
    M: int
    H: int
    prefix: np.ndarray
    add: np.ndarray
    add2: Optional[np.ndarray]
    snapshots: List[np.ndarray]
    query: np.ndarray
    gamma: np.ndarray
    eps: float = EPS

    @property
    def N(self) -> int:
        return len(self.snapshots)

    def algorithmic_bytes(self) -> int:
        """Bytes one call must move: reads prefix, add, [add2], N snapshots,
        writes out_prefix and out_norm (all [M,H] bf16), plus query and gamma."""
        streams = 4 + (1 if self.add2 is not None else 0) + self.N
        return 2 * self.H * (self.M * streams + 2)

    def rows(self, idx: Sequence[int]) -> "Case":
        """The same case restricted to a subset of tokens (tokens are independent)."""
        idx = np.asarray(idx)
        return dataclasses.replace(
            self, M=len(idx), prefix=self.prefix[idx], add=self.add[idx],
            add2=None if self.add2 is None else self.add2[idx],
            snapshots=[s[idx] for s in self.snapshots])


def layer_params(key, H: int):
    query = normal((*key, "query"), (H,), sigma=1.0 / np.sqrt(H))
    gamma = normal((*key, "gamma"), (H,), sigma=0.1, mu=1.0)
    return query, gamma


def make_case(cfg: int, M: int, N: int, add2: bool, H: int = H_MODEL,
              special: Optional[str] = None, name: Optional[str] = None) -> Case:
    """A random call.  ``special`` adds the structure of the named workloads:

    * ``"subnormal"``: 1% of (token, column) pairs get routed/shared addends
      that cancel into a bf16 subnormal sum, 1% of prefix entries become
      random nonzero bf16 subnormals; half of the first set also gets a
      signed-zero prefix and half of the second gets shared = -routed, so the
      subnormals reach the updated prefix;
    * ``"scaled"``: snapshot j is multiplied by 10^u_j, u_j ~ U(-2, 1).
    """
    key = (cfg, M, N, int(add2), H)
    prefix = normal((*key, "prefix"), (M, H))
    if add2:
        add = normal((*key, "routed"), (M, H), sigma=0.5)
        add_2 = normal((*key, "shared"), (M, H), sigma=0.5)
    else:
        add = normal((*key, "add"), (M, H))
        add_2 = None
    snaps = []
    for j in range(N):
        if special == "scaled":
            u = _rng(*key, "scale", j).uniform(-2.0, 1.0)
            x = _rng(*key, "snap", j).standard_normal((M, H)) * 10.0 ** u
            snaps.append(to_bf16_bits(x))
        else:
            snaps.append(normal((*key, "snap", j), (M, H)))
    query, gamma = layer_params(key, H)
    if special == "subnormal":
        if not add2:
            raise ValueError("the subnormal structure needs two addends")
        _plant_subnormals(key, prefix, add, add_2)
    return Case(name or "cfg%d" % cfg, M, H, prefix, add, add_2, snaps, query, gamma)


def _plant_subnormals(key, prefix, routed, shared):
    rng = _rng(*key, "subnormal")
    M, H = prefix.shape
    n = max(2, (M * H) // 100)
    flat = rng.permutation(M * H)
    pair, sub = flat[:n], flat[n:2 * n]
    # routed = (1 + k/128) 2^-126, shared = -2^-126  ->  sum = k 2^-133
    sign = rng.integers(0, 2, n).astype(np.uint16) << 15
    k = rng.integers(1, 128, n).astype(np.uint16)
    r = routed.reshape(-1)
    s = shared.reshape(-1)
    p = prefix.reshape(-1)
    r[pair] = sign | 0x0080 | k
    s[pair] = (sign ^ 0x8000) | 0x0080
    half = pair[: n // 2]
    p[half] = rng.integers(0, 2, len(half)).astype(np.uint16) << 15  # +-0
    # prefix = random nonzero subnormal
    sign2 = rng.integers(0, 2, n).astype(np.uint16) << 15
    p[sub] = sign2 | rng.integers(1, 128, n).astype(np.uint16)
    half2 = sub[: n // 2]
    s[half2] = r[half2] ^ 0x8000  # shared = -routed exactly


# The named workloads ------------------------------------------------------

CONFIGS: Dict[str, dict] = {
    # plain add + AttnRes + RMSNorm, no second addend
    "cfg1": dict(cfg=1, M=1, N=1, add2=False),
    # workgroup-per-token regime
    "cfg2": dict(cfg=2, M=8, N=4, add2=True),
    # split-H regime, with subnormal structure
    "cfg3": dict(cfg=3, M=16, N=8, add2=True, special="subnormal"),
    # the largest fused window, sources of very different magnitudes
    "cfg4": dict(cfg=4, M=32, N=12, add2=True, special="scaled"),
    # single-token call with every source
    "cfg4b": dict(cfg=4, M=1, N=12, add2=True, special="scaled"),
}


def config_case(name: str, H: int = H_MODEL) -> Case:
    kw = dict(CONFIGS[name])
    return make_case(H=H, name=name, **kw)


# The 25-layer decoder chain ---------------------------------------------

CHAIN_LAYERS = 25
CHAIN_TOKENS = 256


@dataclasses.dataclass
class ChainLayer:
    """Inputs of one chain layer and its place in the snapshot-bank schedule."""

    n_sources: int         # bank entries the layer mixes (= bank size at the call)
    push_after: bool       # append the layer's updated prefix to the bank, restart at +0
    query: np.ndarray
    gamma: np.ndarray
    routed: np.ndarray     # the deferred MoE tail folded into this call
    shared: np.ndarray


@dataclasses.dataclass
class Chain:
    M: int
    H: int
    embedding: np.ndarray  # first bank entry
    prefix0: np.ndarray
    layers: List[ChainLayer]
    eps: float = EPS

    def algorithmic_bytes(self) -> int:
        return sum(2 * self.H * (self.M * (5 + l.n_sources) + 2) for l in self.layers)

    def rows(self, idx: Sequence[int]) -> "Chain":
        idx = np.asarray(idx)
        return Chain(len(idx), self.H, self.embedding[idx], self.prefix0[idx], [
            dataclasses.replace(l, routed=l.routed[idx], shared=l.shared[idx])
            for l in self.layers], self.eps)


def chain_schedule(layers: int = CHAIN_LAYERS, max_sources: int = MAX_SOURCES):
    """(n_sources, push_after) per layer.  The bank starts with the embedding;
    after every odd layer the updated prefix is pushed while the bank holds
    fewer than ``max_sources`` entries (and the next prefix restarts at +0),
    otherwise it is carried on."""
    out, bank = [], 1
    for l in range(layers):
        push = (l % 2 == 1) and bank < max_sources
        out.append((bank, push))
        if push:
            bank += 1
    return out


def make_chain(M: int = CHAIN_TOKENS, H: int = H_MODEL, layers: int = CHAIN_LAYERS,
               seed: int = 5) -> Chain:
    emb = normal((seed, "embedding", M, H), (M, H))
    p0 = normal((seed, "prefix0", M, H), (M, H))
    out = []
    for l, (n, push) in enumerate(chain_schedule(layers)):
        q, g = layer_params((seed, l, H), H)
        r = normal((seed, l, "routed", M, H), (M, H), sigma=0.5)
        s = normal((seed, l, "shared", M, H), (M, H), sigma=0.5)
        out.append(ChainLayer(n, push, q, g, r, s))
    return Chain(M, H, emb, p0, out)


def run_chain(chain: Chain, step, fresh_zero, embedding=None, prefix0=None):
    """Drive the chain's hand-off and return ``(outputs, bank)``.

    ``step(layer_index, prefix, bank, layer)`` runs one fused call and returns
    ``(out_prefix, out_norm)``; ``fresh_zero()`` returns a +0 prefix;
    ``embedding``/``prefix0`` override the chain's own arrays (e.g. with device
    copies).  ``outputs`` lists ``(out_prefix, out_norm)`` per layer.  This is
    the hand-off only (which tensor goes where); it holds no arithmetic of the
    operation itself."""
    bank = [chain.embedding if embedding is None else embedding]
    prefix = chain.prefix0 if prefix0 is None else prefix0
    outputs = []
    for l, layer in enumerate(chain.layers):
        assert len(bank) == layer.n_sources
        out_prefix, out_norm = step(l, prefix, list(bank), layer)
        outputs.append((out_prefix, out_norm))
        if layer.push_after:
            bank.append(out_prefix)
            prefix = fresh_zero()
        else:
            prefix = out_prefix
    return outputs, bank
