"""Exact, IO-aware attention forward for AMD Instinct MI355X (gfx950).

The computation lives in the HIP library libexact_attn.so (C ABI declared in
include/exact_attn.h); this package is its thin Python binding.
"""
from .api import (  # noqa: F401
    attn_bwd,
    attn_bwd_workspace_size,
    attn_fwd,
    attn_paged_decode,
    attn_paged_decode_noalloc,
    attn_paged_decode_workspace_size,
    attn_paged_prefill,
)
from ._lib import AttnError, LIB_PATH, lib, status_string  # noqa: F401
