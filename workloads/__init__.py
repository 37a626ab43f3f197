"""Seeded synthetic inputs shared by the oracle-side checks and the HIP-side runs.

This package holds no attention arithmetic: it only draws random numbers,
rounds them to the storage type and lays them out (including the paged KV
cache and its block table).  Both the oracle and the GPU path consume what it
returns; neither of them is imported here.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    bf16_bits_from_f32,
    doc_lengths,
    make_decode,
    make_prefill,
    prefill_config,
    decode_config,
    make_chunked_prefill,
    make_backward,
    chunked_config,
)
