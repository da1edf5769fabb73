"""Batched speculative-sampling verification on AMD Instinct MI355X (gfx950).

The computation lives in libspecv.so (HIP kernels behind a C ABI, declared in
include/specv.h); this package builds it and binds it with ctypes.
"""

from ._lib import (  # noqa: F401
    SPECV_BF16,
    SPECV_EALIGN,
    SPECV_EHIP,
    SPECV_EINVAL,
    SPECV_ENOMEM,
    SPECV_ERANGE,
    SPECV_ESTATE,
    SPECV_F32,
    SPECV_MAX_DRAFT,
    SPECV_OK,
    SpecvError,
    Verifier,
    load_library,
    specv_acceptance_rates,
    specv_create,
    specv_destroy,
    specv_kv_commit,
    specv_last_timings,
    specv_row_stats,
    specv_sample,
    specv_set_timing,
    specv_set_wait_limit,
    specv_stage_name,
    specv_strerror,
    specv_verify,
    specv_verify_lazy,
    specv_verify_static,
)

__all__ = [
    "Verifier",
    "SpecvError",
    "load_library",
    "specv_create",
    "specv_acceptance_rates",
    "specv_verify",
    "specv_verify_lazy",
    "specv_verify_static",
    "specv_row_stats",
    "specv_sample",
    "specv_destroy",
    "specv_kv_commit",
    "specv_strerror",
]
