"""CPU oracle for the fused AttnRes combine + RMSNorm with the MoE-tail fold.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``attention_residual_rmsnorm_amd``) never imports it and shares no code with it.

The arithmetic lives in ``attnres_oracle.c`` (binary32 fold-add, binary64 mix
and RMSNorm, one final rounding); this module only marshals numpy arrays of
bf16 bit patterns (``uint16``) into it through ctypes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f64p = ctypes.POINTER(ctypes.c_double)


def _ptr(a: Optional[np.ndarray], kind=_u16p):
    if a is None:
        return None
    return a.ctypes.data_as(kind)


class Oracle:
    """ctypes view of one build of the oracle library (the real one, or a test mutant)."""

    def __init__(self, path: Optional[str] = None):
        if path is None:
            path = _build.LIBRARY
            if not os.path.exists(path):
                _build.build()
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_add.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        lib.oracle_bf16_add.restype = ctypes.c_uint16
        lib.oracle_bf16_add_tensor.argtypes = [_u16p, _u16p, _u16p, ctypes.c_int64]
        lib.oracle_bf16_add_tensor.restype = None
        lib.oracle_attnres_fwd.argtypes = [
            _u16p, _u16p, _u16p, ctypes.POINTER(_u16p), ctypes.c_int, _u16p, _u16p,
            ctypes.c_float, ctypes.c_int64, ctypes.c_int64, _u16p, _u16p, _f64p, _f64p]
        lib.oracle_attnres_fwd.restype = ctypes.c_int
        lib.oracle_attnres_fwd_mix.argtypes = [
            _u16p, _u16p, _u16p, ctypes.POINTER(_u16p), ctypes.c_int, _u16p, _u16p,
            ctypes.c_float, ctypes.c_int64, ctypes.c_int64, _u16p, _u16p, _u16p, _f64p, _f64p,
            _f64p]
        lib.oracle_attnres_fwd_mix.restype = ctypes.c_int
        self.lib = lib

    # scalar helpers -------------------------------------------------------
    def round_bf16(self, x: float) -> int:
        return int(self.lib.oracle_round_bf16(float(x)))

    def bf16_add(self, a: int, b: int) -> int:
        return int(self.lib.oracle_bf16_add(a, b))

    def add_tensor(self, a: np.ndarray, b: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.uint16)
        b = np.ascontiguousarray(b, dtype=np.uint16)
        assert a.shape == b.shape
        out = np.empty_like(a)
        self.lib.oracle_bf16_add_tensor(_ptr(a), _ptr(b), _ptr(out), a.size)
        return out

    # the fused operation --------------------------------------------------
    def fwd(self, prefix: np.ndarray, add: np.ndarray, add2: Optional[np.ndarray],
            snapshots: Sequence[np.ndarray], query: np.ndarray, gamma: np.ndarray,
            eps: float, want_f64: bool = False, want_alpha: bool = False,
            want_mix: bool = False, want_mix_f64: bool = False):
        """Run the oracle on [M,H] bf16-bit arrays.

        Returns ``(out_prefix, out_norm)`` plus, on request and in this order,
        ``out_norm_f64``, ``alpha`` ([M, N+1], sources in the order snapshots...,
        updated prefix), ``out_mix`` (the pre-norm mixture rounded to bf16) and
        ``out_mix_f64`` (the mixture in binary64).
        """
        prefix = np.ascontiguousarray(prefix, dtype=np.uint16)
        M, H = prefix.shape
        add = np.ascontiguousarray(add, dtype=np.uint16)
        add2 = None if add2 is None else np.ascontiguousarray(add2, dtype=np.uint16)
        snaps = [np.ascontiguousarray(s, dtype=np.uint16) for s in snapshots]
        for t in [add, add2, *snaps]:
            if t is not None and t.shape != (M, H):
                raise ValueError("shape mismatch")
        query = np.ascontiguousarray(query, dtype=np.uint16).reshape(H)
        gamma = np.ascontiguousarray(gamma, dtype=np.uint16).reshape(H)
        N = len(snaps)
        arr = (_u16p * max(N, 1))(*[_ptr(s) for s in snaps])
        out_prefix = np.empty((M, H), np.uint16)
        out_norm = np.empty((M, H), np.uint16)
        f64 = np.empty((M, H), np.float64) if want_f64 else None
        alpha = np.empty((M, N + 1), np.float64) if want_alpha else None
        mix = np.empty((M, H), np.uint16) if want_mix else None
        mix64 = np.empty((M, H), np.float64) if want_mix_f64 else None
        rc = self.lib.oracle_attnres_fwd_mix(
            _ptr(prefix), _ptr(add), _ptr(add2), arr if N else None, N, _ptr(query),
            _ptr(gamma), ctypes.c_float(eps), M, H, _ptr(out_prefix), _ptr(out_norm),
            _ptr(mix), _ptr(f64, _f64p), _ptr(mix64, _f64p), _ptr(alpha, _f64p))
        if rc != 0:
            raise RuntimeError("oracle_attnres_fwd_mix returned %d" % rc)
        res = [out_prefix, out_norm]
        for want, arr_ in ((want_f64, f64), (want_alpha, alpha), (want_mix, mix),
                           (want_mix_f64, mix64)):
            if want:
                res.append(arr_)
        return tuple(res)


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from ``attnres_oracle.c`` (built on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
