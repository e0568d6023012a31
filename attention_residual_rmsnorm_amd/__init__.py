"""MI355X (gfx950) fused AttnRes combine + RMSNorm with the folded MoE-tail add.

The compute lives in ``libattnres.so`` (HIP kernels behind the C ABI declared in
``include/attnres.h``).  This package is a thin ctypes binding with the same
entry-point names: it checks dtypes and shapes, passes ``data_ptr()`` values and
the current torch stream, and turns negative status codes into exceptions.
Every step of the operation runs in the HIP library; there is no fallback, and
calling an entry point without the built library raises immediately.
"""
from ._binding import (  # noqa: F401
    ATTNRES_EALIAS,
    ATTNRES_EHIP,
    ATTNRES_EINVAL,
    ATTNRES_ENOINIT,
    ATTNRES_ESCRATCH,
    ATTNRES_NOALLOC_MAX_SPLIT_TOKENS,
    ATTNRES_EUNSUPPORTED,
    ATTNRES_MAX_HIDDEN,
    ATTNRES_MAX_SNAPSHOTS,
    ATTNRES_OK,
    AttnResError,
    attnres_add_rmsnorm_fwd,
    attnres_add_rmsnorm_fwd_noalloc,
    attnres_add_rmsnorm_mix_fwd,
    attnres_bf16_add,
    attnres_debug_timeouts,
    attnres_debug_set_spin_limit,
    attnres_debug_reset_scratch,
    attnres_debug_set_epoch,
    attnres_debug_set_exchange,
    attnres_debug_set_slot_rotation,
    attnres_init,
    attnres_plan,
    attnres_selftest_rounding,
    attnres_set_variant,
    attnres_status_string,
    attnres_version,
    library,
    library_path,
)
