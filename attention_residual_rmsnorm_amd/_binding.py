"""ctypes binding of libattnres (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

ATTNRES_OK = 0
ATTNRES_EINVAL = -1
ATTNRES_EUNSUPPORTED = -2
ATTNRES_EALIAS = -3
ATTNRES_EHIP = -4
ATTNRES_ENOINIT = -5
ATTNRES_ESCRATCH = -6
ATTNRES_NOALLOC_MAX_SPLIT_TOKENS = 96
ATTNRES_MAX_SNAPSHOTS = 64
ATTNRES_MAX_HIDDEN = 16384

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libattnres.so")

_lib = None
_vp = ctypes.c_void_p


class AttnResError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (where, attnres_status_string(status), status))


def library():
    """Load libattnres.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        # Load torch's HIP runtime first.  libattnres links libamdhip64.so.7;
        # torch ships its own copy under that soname, so when torch is already
        # loaded the dynamic loader binds libattnres to the same runtime that
        # owns the device pointers and stream handles passed in.  Loading
        # libattnres first would put a second HIP runtime in the process.
        import torch  # noqa: F401

        if not os.path.exists(library_path):
            raise ImportError(
                "libattnres.so is not built (expected at %s); run __graft_entry__.build() "
                "or python attention_residual_rmsnorm_amd/build.py" % library_path)
        lib = ctypes.CDLL(library_path)
        lib.attnres_add_rmsnorm_fwd.argtypes = [
            _vp, _vp, _vp, ctypes.POINTER(_vp), ctypes.c_int, _vp, _vp, ctypes.c_float,
            ctypes.c_int64, ctypes.c_int64, _vp, _vp, _vp]
        lib.attnres_add_rmsnorm_fwd.restype = ctypes.c_int
        lib.attnres_add_rmsnorm_mix_fwd.argtypes = [
            _vp, _vp, _vp, ctypes.POINTER(_vp), ctypes.c_int, _vp, _vp, ctypes.c_float,
            ctypes.c_int64, ctypes.c_int64, _vp, _vp, _vp, _vp]
        lib.attnres_add_rmsnorm_mix_fwd.restype = ctypes.c_int
        lib.attnres_add_rmsnorm_fwd_noalloc.argtypes = [
            _vp, _vp, _vp, ctypes.POINTER(_vp), ctypes.c_int, _vp, _vp, ctypes.c_float,
            ctypes.c_int64, ctypes.c_int64, _vp, _vp, _vp]
        lib.attnres_add_rmsnorm_fwd_noalloc.restype = ctypes.c_int
        lib.attnres_bf16_add.argtypes = [_vp, _vp, _vp, ctypes.c_int64, _vp]
        lib.attnres_bf16_add.restype = ctypes.c_int
        lib.attnres_init.argtypes = []
        lib.attnres_init.restype = ctypes.c_int
        lib.attnres_plan.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                     ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                                     ctypes.POINTER(ctypes.c_int)]
        lib.attnres_plan.restype = ctypes.c_int
        lib.attnres_set_variant.argtypes = [ctypes.c_int, ctypes.c_int]
        lib.attnres_set_variant.restype = ctypes.c_int
        lib.attnres_debug_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint)]
        lib.attnres_debug_timeouts.restype = ctypes.c_int
        lib.attnres_debug_set_spin_limit.argtypes = [ctypes.c_uint]
        lib.attnres_debug_set_spin_limit.restype = ctypes.c_int
        lib.attnres_debug_reset_scratch.argtypes = []
        lib.attnres_debug_reset_scratch.restype = ctypes.c_int
        lib.attnres_debug_set_epoch.argtypes = [ctypes.c_uint]
        lib.attnres_debug_set_epoch.restype = ctypes.c_int
        lib.attnres_debug_set_exchange.argtypes = [ctypes.c_int]
        lib.attnres_debug_set_exchange.restype = ctypes.c_int
        lib.attnres_debug_set_slot_rotation.argtypes = [ctypes.c_int]
        lib.attnres_debug_set_slot_rotation.restype = ctypes.c_int
        lib.attnres_selftest_rounding.argtypes = [ctypes.POINTER(ctypes.c_ulonglong)]
        lib.attnres_selftest_rounding.restype = ctypes.c_int
        lib.attnres_status_string.argtypes = [ctypes.c_int]
        lib.attnres_status_string.restype = ctypes.c_char_p
        lib.attnres_version.argtypes = []
        lib.attnres_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(rc: int, where: str) -> None:
    if rc != ATTNRES_OK:
        raise AttnResError(rc, where)


_initialised = set()


def _ensure_init() -> None:
    """attnres_init() on the current device before the binding's first fused
    call there (the library requires it; it allocates the device's scratch
    and synchronises, once).  Callers that must not allocate at that point
    (HIP-graph capture) call attnres_init() themselves beforehand."""
    import torch

    dev = torch.cuda.current_device()
    if dev not in _initialised:
        _check(library().attnres_init(), "attnres_init")
        _initialised.add(dev)


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (or a raw integer address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check_tensor(name, t, shape):
    import torch

    if t.dtype != torch.bfloat16:
        raise TypeError("%s must be bfloat16, got %s" % (name, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)


def _fwd_args(prefix, add, add2, snapshots, query, gamma, out_prefix, out_norm):
    import torch

    M, H = prefix.shape
    for name, t in (("prefix", prefix), ("add", add)):
        _check_tensor(name, t, (M, H))
    if add2 is not None:
        _check_tensor("add2", add2, (M, H))
    for i, s in enumerate(snapshots):
        _check_tensor("snapshots[%d]" % i, s, (M, H))
    _check_tensor("query", query, (H,))
    _check_tensor("gamma", gamma, (H,))
    if out_prefix is None:
        out_prefix = torch.empty_like(prefix)
    if out_norm is None:
        out_norm = torch.empty_like(prefix)
    _check_tensor("out_prefix", out_prefix, (M, H))
    _check_tensor("out_norm", out_norm, (M, H))
    n = len(snapshots)
    arr = (_vp * max(n, 1))(*[_ptr(s) for s in snapshots])
    return M, H, n, arr, out_prefix, out_norm


def attnres_add_rmsnorm_fwd(prefix, add, add2, snapshots: Sequence, query, gamma, eps: float,
                            out_prefix=None, out_norm=None, stream=None):
    """Fused fold-add + AttnRes mix + RMSNorm on bf16 device tensors.

    prefix, add, add2 (or None), each snapshot, out_prefix, out_norm: [M, H];
    query, gamma: [H].  Outputs are allocated when not given.  Returns
    ``(out_prefix, out_norm)``.  Runs on the current torch stream unless
    ``stream`` (a torch stream or raw handle) is given.
    """
    M, H, n, arr, out_prefix, out_norm = _fwd_args(prefix, add, add2, snapshots, query, gamma,
                                                   out_prefix, out_norm)
    _ensure_init()
    rc = library().attnres_add_rmsnorm_fwd(
        _ptr(prefix), _ptr(add), _ptr(add2), arr if n else None, n, _ptr(query), _ptr(gamma),
        ctypes.c_float(eps), M, H, _ptr(out_prefix), _ptr(out_norm), _stream(stream))
    _check(rc, "attnres_add_rmsnorm_fwd")
    return out_prefix, out_norm


def attnres_add_rmsnorm_fwd_noalloc(prefix, add, add2, snapshots: Sequence, query, gamma, eps: float,
                                    out_prefix, out_norm, stream=None):
    """attnres_add_rmsnorm_fwd for callers that cannot allocate: the library
    allocates nothing (its split-kernel scratch is a static device array) and
    needs no attnres_init.  The outputs must be given (this wrapper allocates
    nothing either).  Returns ``(out_prefix, out_norm)``."""
    M, H, n, arr, out_prefix, out_norm = _fwd_args(prefix, add, add2, snapshots, query, gamma,
                                                   out_prefix, out_norm)
    rc = library().attnres_add_rmsnorm_fwd_noalloc(
        _ptr(prefix), _ptr(add), _ptr(add2), arr if n else None, n, _ptr(query), _ptr(gamma),
        ctypes.c_float(eps), M, H, _ptr(out_prefix), _ptr(out_norm), _stream(stream))
    _check(rc, "attnres_add_rmsnorm_fwd_noalloc")
    return out_prefix, out_norm


def attnres_add_rmsnorm_mix_fwd(prefix, add, add2, snapshots: Sequence, query, gamma, eps: float,
                                out_prefix=None, out_norm=None, out_mix=None, stream=None):
    """attnres_add_rmsnorm_fwd plus the pre-norm mixture (bf16 [M, H], for a
    hidden-state capture tap).  Returns ``(out_prefix, out_norm, out_mix)``."""
    import torch

    M, H, n, arr, out_prefix, out_norm = _fwd_args(prefix, add, add2, snapshots, query, gamma,
                                                   out_prefix, out_norm)
    if out_mix is None:
        out_mix = torch.empty_like(prefix)
    _check_tensor("out_mix", out_mix, (M, H))
    _ensure_init()
    rc = library().attnres_add_rmsnorm_mix_fwd(
        _ptr(prefix), _ptr(add), _ptr(add2), arr if n else None, n, _ptr(query), _ptr(gamma),
        ctypes.c_float(eps), M, H, _ptr(out_prefix), _ptr(out_norm), _ptr(out_mix), _stream(stream))
    _check(rc, "attnres_add_rmsnorm_mix_fwd")
    return out_prefix, out_norm, out_mix


def attnres_bf16_add(a, b, out=None, stream=None):
    """out = bf16(a + b) elementwise on bf16 device tensors (the unfused tail add)."""
    import torch

    _check_tensor("a", a, a.shape)
    _check_tensor("b", b, a.shape)
    if out is None:
        out = torch.empty_like(a)
    _check_tensor("out", out, a.shape)
    _check(library().attnres_bf16_add(_ptr(a), _ptr(b), _ptr(out), a.numel(), _stream(stream)),
           "attnres_bf16_add")
    return out


def attnres_init() -> None:
    """Allocate the current device's scratch (synchronously; once per device)."""
    import torch

    _check(library().attnres_init(), "attnres_init")
    _initialised.add(torch.cuda.current_device())


def attnres_plan(M: int, n_snapshots: int, H: int):
    """(variant, chunks, threads) the fused call would launch with."""
    v, c, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(library().attnres_plan(M, n_snapshots, H, ctypes.byref(v), ctypes.byref(c), ctypes.byref(t)),
           "attnres_plan")
    return v.value, c.value, t.value


def attnres_set_variant(variant: int, param: int = 0) -> None:
    _check(library().attnres_set_variant(variant, param), "attnres_set_variant")


def attnres_debug_timeouts() -> int:
    out = ctypes.c_uint()
    _check(library().attnres_debug_timeouts(ctypes.byref(out)), "attnres_debug_timeouts")
    return out.value


def attnres_debug_set_spin_limit(limit: int = 0) -> None:
    _check(library().attnres_debug_set_spin_limit(limit), "attnres_debug_set_spin_limit")


def attnres_debug_set_exchange(mode: int = 0) -> None:
    _check(library().attnres_debug_set_exchange(mode), "attnres_debug_set_exchange")


def attnres_debug_set_slot_rotation(on: bool = True) -> None:
    _check(library().attnres_debug_set_slot_rotation(1 if on else 0), "attnres_debug_set_slot_rotation")


def attnres_debug_reset_scratch() -> None:
    _check(library().attnres_debug_reset_scratch(), "attnres_debug_reset_scratch")


def attnres_debug_set_epoch(epoch: int) -> None:
    _check(library().attnres_debug_set_epoch(epoch), "attnres_debug_set_epoch")


def attnres_selftest_rounding() -> int:
    """Number of binary32 inputs whose device bf16 rounding disagrees with the
    definition (0 expected); runs on the current device."""
    out = ctypes.c_ulonglong()
    _check(library().attnres_selftest_rounding(ctypes.byref(out)), "attnres_selftest_rounding")
    return out.value


def attnres_status_string(status: int) -> str:
    try:
        return library().attnres_status_string(status).decode()
    except ImportError:
        return "status %d" % status


def attnres_version() -> int:
    return library().attnres_version()
