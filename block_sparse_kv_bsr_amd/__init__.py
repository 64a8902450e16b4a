"""Paged / block-sparse-row (BSR) GQA decode attention for AMD MI355X.

The compute path is the C-ABI library ``libfi_bsr.so`` (HIP kernels for
gfx950, declared in include/fi_bsr.h); this package is its ctypes binding
plus seeded input generators. ``plan``, ``decode``, ``merge_states``,
``prefill_plan``, ``prefill``, ``mla_plan`` and ``mla`` load the library on first use and raise if it
is missing.
"""
from .binding import (FiError, Plan, PrefillPlan, decode, decode_composed,  # noqa: F401
                      decode_noalloc, lib, merge_states, mla, mla_plan, plan, plan_composed,
                      prefill, prefill_plan, FI_DTYPE_BF16, FI_DTYPE_F32, FI_DTYPE_FP8_E4M3)
