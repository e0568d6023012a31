"""Comparator and device helpers shared by the GPU parity tests.

Accuracy bar:
  * out_prefix: bit-exact (16-bit patterns equal);
  * out_norm: per element, within 2 bf16 ulps (distance between the patterns
    mapped to a monotone integer scale, so it counts across binade edges and
    treats +0 and -0 alike) OR within 1e-2 absolute; any NaN fails.
The 2-ulp bound comes from the arithmetic: the device mixes and normalises in
binary32 (relative error well below 2^-16 for these sizes) and rounds once to
bf16 (<= 1/2 ulp), against a binary64 reference rounded once (<= 1/2 ulp).
"""
from __future__ import annotations

import numpy as np

from attention_residual_rmsnorm_amd import workloads as W

ULP_TOL = 2
ABS_TOL = 1e-2


def ord16(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def is_nan16(bits) -> np.ndarray:
    b = np.asarray(bits, np.uint16)
    return ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)


def norm_mismatches(got: np.ndarray, want: np.ndarray):
    """Boolean mask of out_norm elements outside the accuracy bar."""
    got = np.asarray(got, np.uint16)
    want = np.asarray(want, np.uint16)
    ulps = np.abs(ord16(got) - ord16(want))
    diff = np.abs(W.bf16_bits_to_f32(got).astype(np.float64) - W.bf16_bits_to_f32(want).astype(np.float64))
    ok = (ulps <= ULP_TOL) | (diff <= ABS_TOL)
    ok &= ~is_nan16(got) & ~is_nan16(want)
    return ~ok


def assert_parity(gpu_prefix, gpu_norm, ref_prefix, ref_norm, what=""):
    gpu_prefix = np.asarray(gpu_prefix, np.uint16)
    ref_prefix = np.asarray(ref_prefix, np.uint16)
    bad = np.argwhere(gpu_prefix != ref_prefix)
    assert bad.size == 0, "%s: out_prefix differs at %d places, first %s: gpu %04x oracle %04x" % (
        what, len(bad), tuple(bad[0]), gpu_prefix[tuple(bad[0])], ref_prefix[tuple(bad[0])])
    mask = norm_mismatches(gpu_norm, ref_norm)
    if mask.any():
        i = tuple(np.argwhere(mask)[0])
        g, r = np.asarray(gpu_norm)[i], np.asarray(ref_norm)[i]
        raise AssertionError("%s: out_norm outside 2 ulps / 1e-2 at %d places, first %s: gpu %04x (%g) "
                             "oracle %04x (%g)" % (what, int(mask.sum()), i, g, W.bf16_bits_to_f32(np.array([g]))[0],
                                                   r, W.bf16_bits_to_f32(np.array([r]))[0]))


def max_ulps(gpu_norm, ref_norm) -> int:
    return int(np.max(np.abs(ord16(gpu_norm) - ord16(ref_norm)))) if np.size(gpu_norm) else 0


# device transfer ----------------------------------------------------------

def dev(bits: np.ndarray, device="cuda"):
    """numpy bf16 bits -> torch bfloat16 device tensor."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def host(t) -> np.ndarray:
    import torch

    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16).copy()


def run_gpu(case: W.Case, add2=True, out_prefix=None, out_norm=None):
    """Run the fused call on a workload case; returns numpy (out_prefix, out_norm)."""
    import attention_residual_rmsnorm_amd as ar

    d = lambda x: None if x is None else dev(x)
    op, on = ar.attnres_add_rmsnorm_fwd(
        d(case.prefix), d(case.add), d(case.add2) if add2 else None, [d(s) for s in case.snapshots],
        d(case.query), d(case.gamma), case.eps, out_prefix=out_prefix, out_norm=out_norm)
    return host(op), host(on)


def run_oracle(orc, case: W.Case):
    return orc.fwd(case.prefix, case.add, case.add2, case.snapshots, case.query, case.gamma, case.eps)


def run_gpu_mix(case: W.Case):
    """The fused call with the pre-norm mixture output; numpy (out_prefix, out_norm, out_mix)."""
    import attention_residual_rmsnorm_amd as ar

    d = lambda x: None if x is None else dev(x)
    op, on, om = ar.attnres_add_rmsnorm_mix_fwd(
        d(case.prefix), d(case.add), d(case.add2), [d(s) for s in case.snapshots],
        d(case.query), d(case.gamma), case.eps)
    return host(op), host(on), host(om)


def run_oracle_mix(orc, case: W.Case):
    """Oracle (out_prefix, out_norm, out_mix)."""
    return orc.fwd(case.prefix, case.add, case.add2, case.snapshots, case.query, case.gamma, case.eps,
                   want_mix=True)


def assert_mix_parity(gpu_mix, ref_mix, what=""):
    """The mixture has out_norm's bar: 2 bf16 ulps or 1e-2 absolute, no NaN."""
    mask = norm_mismatches(gpu_mix, ref_mix)
    if mask.any():
        i = tuple(np.argwhere(mask)[0])
        raise AssertionError("%s: out_mix outside 2 ulps / 1e-2 at %d places, first %s: gpu %04x oracle %04x"
                             % (what, int(mask.sum()), i, np.asarray(gpu_mix)[i], np.asarray(ref_mix)[i]))
