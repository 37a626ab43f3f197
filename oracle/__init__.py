"""fp64 CPU oracle for exact attention (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The HIP library never does, and this package imports
nothing from it.
"""
from .attention import (  # noqa: F401
    MASKS,
    attention,
    from_bf16_bits,
    gather_sequence,
    paged_decode,
    paged_prefill,
    round_to_bf16,
    attention_backward,
    to_f64,
    visibility,
)
