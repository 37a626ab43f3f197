"""Python binding over the C ABI (same names, torch tensors in, torch tensors out).

The functions only check tensor metadata, allocate outputs with torch and pass
raw device pointers plus torch's current HIP stream to the library; every
step of the computation runs in the library's kernels.
"""
from __future__ import annotations

import math

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.ATTN_DTYPE_BF16, torch.float32: _lib.ATTN_DTYPE_F32}


def ctypes_ptr(t: torch.Tensor):
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _check_buffer(t: torch.Tensor, name: str, shape, dtype, device):
    """A caller-supplied output or scratch tensor must be exactly what the
    kernels write: the library sees only a pointer and cannot check it."""
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _need(t.device == device, f"{name} must be on {device}, got {t.device}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _workspace_bytes(ws: torch.Tensor, device) -> int:
    _need(isinstance(ws, torch.Tensor) and ws.device == device and ws.is_contiguous(),
          f"workspace must be a contiguous tensor on {device}")
    return ws.numel() * ws.element_size()


def _same_device(device, *ts):
    _need(all(t.device == device for t in ts), f"every tensor must be on {device}")


def _sink_ptr(sink_logits: torch.Tensor | None, Hq: int):
    if sink_logits is None:
        return None
    _need(sink_logits.dtype == torch.float32 and sink_logits.is_cuda and sink_logits.is_contiguous()
          and sink_logits.numel() == Hq, "sink_logits must be a contiguous float32 device tensor of Hq entries")
    return sink_logits.data_ptr()


def _slopes_ptr(alibi_slopes: torch.Tensor | None, Hq: int):
    if alibi_slopes is None:
        return None
    _need(alibi_slopes.dtype == torch.float32 and alibi_slopes.is_cuda and alibi_slopes.is_contiguous()
          and alibi_slopes.numel() == Hq, "alibi_slopes must be a contiguous float32 device tensor of Hq entries")
    return alibi_slopes.data_ptr()


def make_mask(mask: str = "none", window: int = 0, doc_offsets: torch.Tensor | None = None,
              sink_tokens: int = 0, sink_logits: torch.Tensor | None = None, Hq: int = 0,
              softcap: float = 0.0, alibi_slopes: torch.Tensor | None = None,
              soft_exp2: int = 0) -> _lib.AttnMask:
    _need(mask in _lib.MASK_KINDS, f"unknown mask {mask!r}")
    m = _lib.AttnMask()
    m.kind = _lib.MASK_KINDS[mask]
    m.window = int(window) if mask == "window" else 0
    m.sink_tokens = int(sink_tokens)
    m.sink_logits = _sink_ptr(sink_logits, Hq)
    m.softcap = float(softcap)
    m.alibi_slopes = _slopes_ptr(alibi_slopes, Hq)
    m.soft_exp2 = int(soft_exp2)
    if mask == "document":
        _need(doc_offsets is not None and doc_offsets.dtype == torch.int32 and doc_offsets.is_cuda
              and doc_offsets.is_contiguous(), "document mask needs int32 device doc_offsets")
        m.doc_offsets = doc_offsets.data_ptr()
        m.num_docs = doc_offsets.numel() - 1
    else:
        m.doc_offsets = None
        m.num_docs = 0
    return m


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: float | None = None,
             mask: str = "none", window: int = 0, doc_offsets: torch.Tensor | None = None,
             sink_tokens: int = 0, sink_logits: torch.Tensor | None = None,
             softcap: float = 0.0, alibi_slopes: torch.Tensor | None = None,
             out: torch.Tensor | None = None, lse: torch.Tensor | None = None, with_lse: bool = True,
             soft_exp2: int = 0, stream=None):
    """Attention forward: q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] -> (o [B,Hq,Nq,d], lse [B,Hq,Nq] fp32).
    sink_tokens (window mask) and sink_logits [Hq] fp32 are the optional attention sinks;
    softcap and alibi_slopes [Hq] fp32 the optional score modifications (bf16 only).
    soft_exp2 (0, 2 or 4; bf16, d = 128, no score modifications): that many of every 8
    softmax weights take a software 2^x on the FMA units instead of the hardware one."""
    _need(q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-d [B, H, N, d]")
    _need(q.dtype in _DTYPES and k.dtype == q.dtype and v.dtype == q.dtype, "dtype must be bf16 or fp32, same for q/k/v")
    _need(all(t.is_cuda and t.is_contiguous() for t in (q, k, v)), "q, k, v must be contiguous device tensors")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _need(k.shape == v.shape and k.shape[0] == B and k.shape[3] == d, "k/v shape mismatch")
    _same_device(q.device, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if lse is None and with_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buffer(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    m = make_mask(mask, window, doc_offsets, sink_tokens, sink_logits, Hq, softcap, alibi_slopes, soft_exp2)
    st = _lib.lib().attn_fwd(ctypes_ptr(q), ctypes_ptr(k), ctypes_ptr(v), ctypes_ptr(out),
                             None if lse is None else ctypes_ptr(lse),
                             B, Hq, Hkv, Nq, Nk, d, float(scale), m, _DTYPES[q.dtype], _stream(stream))
    _lib.check(st)
    return out, lse


def attn_paged_decode_workspace_size(num_seqs: int, Hq: int, d: int, max_seq_len: int) -> int:
    return int(_lib.lib().attn_paged_decode_workspace_size(num_seqs, Hq, d, max_seq_len))


def attn_paged_decode(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                      block_table: torch.Tensor, seq_lens: torch.Tensor, *, max_seq_len: int,
                      scale: float | None = None, sink_logits: torch.Tensor | None = None,
                      softcap: float = 0.0, alibi_slopes: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                      with_lse: bool = True, stream=None):
    """Paged decode: q [S,Hq,d], pages [P,Hkv,16,d] -> (o [S,Hq,d] bf16, lse [S,Hq] fp32).
    softcap and alibi_slopes [Hq] fp32 are the optional score modifications."""
    _need(q.dim() == 3 and k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "bad shapes")
    _need(q.dtype == torch.bfloat16 and k_pages.dtype == torch.bfloat16 and v_pages.dtype == torch.bfloat16,
          "paged decode is bf16")
    _need(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32, "block_table/seq_lens must be int32")
    _need(all(t.is_cuda and t.is_contiguous() for t in (q, k_pages, v_pages, block_table, seq_lens)),
          "inputs must be contiguous device tensors")
    S, Hq, d = q.shape
    _, Hkv, page_size, _ = k_pages.shape
    _need(block_table.dim() == 2 and block_table.shape[0] == S and seq_lens.shape == (S,), "index shapes")
    _same_device(q.device, k_pages, v_pages, block_table, seq_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = attn_paged_decode_workspace_size(S, Hq, d, max_seq_len)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = _workspace_bytes(workspace, q.device)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if lse is None and with_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buffer(lse, "lse", (S, Hq), torch.float32, q.device)
    st = _lib.lib().attn_paged_decode(ctypes_ptr(q), ctypes_ptr(k_pages), ctypes_ptr(v_pages),
                                      ctypes_ptr(block_table), ctypes_ptr(seq_lens), ctypes_ptr(out),
                                      None if lse is None else ctypes_ptr(lse),
                                      S, Hq, Hkv, d, page_size, block_table.shape[1], int(max_seq_len),
                                      float(scale), _sink_ptr(sink_logits, Hq), float(softcap),
                                      _slopes_ptr(alibi_slopes, Hq), ctypes_ptr(workspace),
                                      ws_bytes, _stream(stream))
    _lib.check(st)
    return out, lse


def attn_paged_decode_noalloc(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                              block_table: torch.Tensor, seq_lens: torch.Tensor, *, max_seq_len: int,
                              scale: float | None = None, sink_logits: torch.Tensor | None = None,
                              softcap: float = 0.0, alibi_slopes: torch.Tensor | None = None,
                              out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                              with_lse: bool = True, stream=None):
    """attn_paged_decode without a workspace: the library's own device scratch
    array holds the partials (calls that overlap on one GPU race).  Pass out=
    and lse= to keep the call free of allocations."""
    _need(q.dim() == 3 and k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "bad shapes")
    _need(q.dtype == torch.bfloat16 and k_pages.dtype == torch.bfloat16 and v_pages.dtype == torch.bfloat16,
          "paged decode is bf16")
    _need(block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32, "block_table/seq_lens must be int32")
    _need(all(t.is_cuda and t.is_contiguous() for t in (q, k_pages, v_pages, block_table, seq_lens)),
          "inputs must be contiguous device tensors")
    S, Hq, d = q.shape
    _, Hkv, page_size, _ = k_pages.shape
    _need(block_table.dim() == 2 and block_table.shape[0] == S and seq_lens.shape == (S,), "index shapes")
    _same_device(q.device, k_pages, v_pages, block_table, seq_lens)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if lse is None and with_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buffer(lse, "lse", (S, Hq), torch.float32, q.device)
    st = _lib.lib().attn_paged_decode_noalloc(ctypes_ptr(q), ctypes_ptr(k_pages), ctypes_ptr(v_pages),
                                              ctypes_ptr(block_table), ctypes_ptr(seq_lens), ctypes_ptr(out),
                                              None if lse is None else ctypes_ptr(lse),
                                              S, Hq, Hkv, d, page_size, block_table.shape[1], int(max_seq_len),
                                              float(scale), _sink_ptr(sink_logits, Hq), float(softcap),
                                              _slopes_ptr(alibi_slopes, Hq), _stream(stream))
    _lib.check(st)
    return out, lse


def attn_paged_prefill(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                       block_table: torch.Tensor, seq_lens: torch.Tensor, q_offsets: torch.Tensor, *,
                       max_seq_len: int, max_q_len: int, scale: float | None = None, mask: str = "causal",
                       window: int = 0, sink_tokens: int = 0, sink_logits: torch.Tensor | None = None,
                       softcap: float = 0.0, alibi_slopes: torch.Tensor | None = None,
                       out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                       with_lse: bool = True, stream=None):
    """Chunked prefill over the paged cache: q [T,Hq,d] token-major, pages [P,Hkv,16,d],
    q_offsets [S+1] -> (o [T,Hq,d] bf16, lse [T,Hq] fp32)."""
    _need(q.dim() == 3 and k_pages.dim() == 4 and v_pages.shape == k_pages.shape, "bad shapes")
    _need(q.dtype == torch.bfloat16 and k_pages.dtype == torch.bfloat16 and v_pages.dtype == torch.bfloat16,
          "paged prefill is bf16")
    _need(all(t.dtype == torch.int32 for t in (block_table, seq_lens, q_offsets)),
          "block_table/seq_lens/q_offsets must be int32")
    _need(all(t.is_cuda and t.is_contiguous() for t in (q, k_pages, v_pages, block_table, seq_lens, q_offsets)),
          "inputs must be contiguous device tensors")
    T, Hq, d = q.shape
    _, Hkv, page_size, _ = k_pages.shape
    S = seq_lens.shape[0]
    _need(block_table.dim() == 2 and block_table.shape[0] == S and q_offsets.shape == (S + 1,), "index shapes")
    _same_device(q.device, k_pages, v_pages, block_table, seq_lens, q_offsets)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_buffer(out, "out", q.shape, q.dtype, q.device)
    if lse is None and with_lse:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check_buffer(lse, "lse", (T, Hq), torch.float32, q.device)
    m = make_mask(mask, window, None, sink_tokens, sink_logits, Hq, softcap, alibi_slopes)
    st = _lib.lib().attn_paged_prefill(ctypes_ptr(q), ctypes_ptr(k_pages), ctypes_ptr(v_pages),
                                       ctypes_ptr(block_table), ctypes_ptr(seq_lens), ctypes_ptr(q_offsets),
                                       ctypes_ptr(out), None if lse is None else ctypes_ptr(lse),
                                       S, Hq, Hkv, d, page_size, block_table.shape[1], int(max_seq_len),
                                       int(max_q_len), float(scale), m, _stream(stream))
    _lib.check(st)
    return out, lse


def attn_bwd_workspace_size(B: int, Hq: int, Nq: int) -> int:
    return int(_lib.lib().attn_bwd_workspace_size(B, Hq, Nq))


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, do: torch.Tensor,
             lse: torch.Tensor, *, scale: float | None = None, mask: str = "none", window: int = 0,
             doc_offsets: torch.Tensor | None = None, sink_tokens: int = 0,
             sink_logits: torch.Tensor | None = None, softcap: float = 0.0,
             alibi_slopes: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Attention backward from the forward's o and lse: -> (dq, dk, dv, dsink); dsink is None
    without sink_logits.  bf16 or fp32 (all five tensors alike), d = 64 or 128; dk/dv sum over
    each KV head's query heads."""
    _need(all(t.dim() == 4 for t in (q, k, v, o, do)), "q, k, v, o, do must be 4-d")
    _need(all(t.dtype == q.dtype for t in (k, v, o, do)) and q.dtype in (torch.bfloat16, torch.float32),
          "q, k, v, o, do must all be bf16 or all float32")
    _need(lse.dtype == torch.float32, "lse must be float32")
    _need(all(t.is_cuda and t.is_contiguous() for t in (q, k, v, o, do, lse)), "inputs must be contiguous device tensors")
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _need(o.shape == q.shape and do.shape == q.shape and lse.shape == (B, Hq, Nq) and v.shape == k.shape, "shapes")
    _same_device(q.device, k, v, o, do, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dsink = None if sink_logits is None else torch.empty(Hq, dtype=torch.float32, device=q.device)
    need = attn_bwd_workspace_size(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = _workspace_bytes(workspace, q.device)
    m = make_mask(mask, window, doc_offsets, sink_tokens, sink_logits, Hq, softcap, alibi_slopes)
    st = _lib.lib().attn_bwd(ctypes_ptr(q), ctypes_ptr(k), ctypes_ptr(v), ctypes_ptr(o), ctypes_ptr(do),
                             ctypes_ptr(lse), ctypes_ptr(dq), ctypes_ptr(dk), ctypes_ptr(dv),
                             None if dsink is None else ctypes_ptr(dsink), B, Hq, Hkv, Nq, Nk, d, float(scale), m,
                             _lib.ATTN_DTYPE_BF16 if q.dtype == torch.bfloat16 else _lib.ATTN_DTYPE_F32,
                             ctypes_ptr(workspace), ws_bytes, _stream(stream))
    _lib.check(st)
    return dq, dk, dv, dsink
