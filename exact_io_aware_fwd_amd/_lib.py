"""ctypes loader for libexact_attn.so (argument marshalling only).

The library is built in-tree by ``exact_io_aware_fwd_amd.build``.  Loading
fails loudly when it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libexact_attn.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARGUMENT = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_WORKSPACE_TOO_SMALL = 3
ATTN_ERR_HIP = 4

ATTN_DTYPE_F32 = 0
ATTN_DTYPE_BF16 = 1

MASK_KINDS = {"none": 0, "causal": 1, "window": 2, "document": 3}


class AttnMask(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("window", ctypes.c_int32),
                ("doc_offsets", ctypes.c_void_p), ("num_docs", ctypes.c_int32),
                ("sink_tokens", ctypes.c_int32), ("sink_logits", ctypes.c_void_p),
                ("softcap", ctypes.c_float), ("alibi_slopes", ctypes.c_void_p),
                ("soft_exp2", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_fwd_amd.build` "
                           "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    i, p, f, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    L.attn_fwd.argtypes = [p, p, p, p, p, i, i, i, i, i, i, f, AttnMask, i, p]
    L.attn_fwd.restype = i
    L.attn_paged_decode_workspace_size.argtypes = [i, i, i, i]
    L.attn_paged_decode_workspace_size.restype = sz
    L.attn_paged_decode.argtypes = [p, p, p, p, p, p, p, i, i, i, i, i, i, i, f, p, f, p, p, sz, p]
    L.attn_paged_decode.restype = i
    L.attn_paged_decode_noalloc.argtypes = [p, p, p, p, p, p, p, i, i, i, i, i, i, i, f, p, f, p, p]
    L.attn_paged_decode_noalloc.restype = i
    L.attn_paged_prefill.argtypes = [p, p, p, p, p, p, p, p, i, i, i, i, i, i, i, i, f, AttnMask, p]
    L.attn_paged_prefill.restype = i
    L.attn_bwd_workspace_size.argtypes = [i, i, i]
    L.attn_bwd_workspace_size.restype = sz
    L.attn_bwd.argtypes = [p, p, p, p, p, p, p, p, p, p, i, i, i, i, i, i, f, AttnMask, i, p, sz, p]
    L.attn_bwd.restype = i
    L.attn_status_string.argtypes = [i]
    L.attn_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().attn_status_string(status).decode()


class AttnError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"attention library returned {status}: {status_string(status)}")
        self.status = status


def check(status: int) -> None:
    if status != ATTN_OK:
        raise AttnError(status)
