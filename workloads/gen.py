"""Seeded generators for the attention workloads.

Every array is drawn from ``numpy.random.default_rng(seed)`` in a fixed order:
structure first (document lengths, context lengths, page permutation), then
Q, K and V, each as float32 standard normals.  bf16 workloads are rounded to
bf16 with round-to-nearest-even and handed out as raw ``uint16`` bit patterns,
so the GPU side can view them as bf16 without another rounding and the
oracle side can widen them exactly.

Shapes follow the layouts of the C ABI:
  prefill  q [B, Hq, Nq, d], k/v [B, Hkv, Nk, d]
  decode   q [S, Hq, d], k_pages/v_pages [P, Hkv, page_size, d],
           block_table [S, max_pages_per_seq] (int32, unused = -1),
           seq_lens [S] (int32)
"""
from __future__ import annotations

import math

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)

# Named workloads.  Sizes are the ones the attention pages use as examples:
# a Llama-3-8B-like head layout (32 query heads, 8 KV heads, head dim 128),
# long contexts, and a 16-token paged KV cache.
CONFIGS = {
    "c1_f32_single_head": dict(kind="prefill", B=1, Hq=1, Hkv=1, Nq=256, Nk=256, d=64,
                               dtype="f32", mask="none"),
    "c2_causal_b4h16n2048": dict(kind="prefill", B=4, Hq=16, Hkv=16, Nq=2048, Nk=2048, d=128,
                                 dtype="bf16", mask="causal"),
    "c3a_gqa_causal_n8192": dict(kind="prefill", B=1, Hq=32, Hkv=8, Nq=8192, Nk=8192, d=128,
                                 dtype="bf16", mask="causal"),
    "c3b_gqa_window1024_n8192": dict(kind="prefill", B=1, Hq=32, Hkv=8, Nq=8192, Nk=8192, d=128,
                                     dtype="bf16", mask="window", window=1024),
    "c4_document_n32768": dict(kind="prefill", B=1, Hq=32, Hkv=8, Nq=32768, Nk=32768, d=128,
                               dtype="bf16", mask="document", doc_min=512, doc_max=8192),
    "c5_paged_decode_64": dict(kind="decode", num_seqs=64, Hq=32, Hkv=8, d=128, page_size=16,
                               len_min=1024, len_max=32768),
}


def bf16_bits_from_f32(x: np.ndarray, chunk: int = 1 << 24) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    NaN inputs map to the canonical quiet NaN.  Works in chunks so that very
    large arrays do not need several full-size temporaries.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    for s in range(0, flat.size, chunk):
        b = flat[s:s + chunk].view(np.uint32)
        rounded = (b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
        r16 = rounded.astype(np.uint16)
        nan = np.isnan(flat[s:s + chunk])
        if nan.any():
            r16[nan] = BF16_QNAN
        out[s:s + chunk] = r16
    return out.reshape(x.shape)


def _draw(rng: np.random.Generator, shape, dtype: str):
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    raise ValueError(f"unknown dtype {dtype}")


def doc_lengths(rng: np.random.Generator, total: int, lo: int, hi: int) -> list[int]:
    """Document lengths drawn uniformly in [lo, hi] until they fill ``total``.

    The last document is cut so the lengths sum to exactly ``total`` (so it
    may be shorter than ``lo``).
    """
    lens: list[int] = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return lens


def make_prefill(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, *, dtype: str = "bf16",
                 seed: int = 0, mask: str = "none", window: int = 0,
                 doc_lens: list[int] | None = None, doc_min: int = 0, doc_max: int = 0,
                 scale: float | None = None) -> dict:
    """Draw one prefill problem.

    ``mask`` is one of none / causal / window / document.  For the document
    mask either pass ``doc_lens`` (summing to Nk) or ``doc_min``/``doc_max``
    to draw them from the seed before Q, K, V.
    """
    rng = np.random.default_rng(seed)
    offsets = None
    if mask == "document":
        if doc_lens is None:
            doc_lens = doc_lengths(rng, Nk, doc_min, doc_max)
        assert sum(doc_lens) == Nk
        offsets = np.concatenate([[0], np.cumsum(doc_lens)]).astype(np.int32)
    q = _draw(rng, (B, Hq, Nq, d), dtype)
    k = _draw(rng, (B, Hkv, Nk, d), dtype)
    v = _draw(rng, (B, Hkv, Nk, d), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return dict(kind="prefill", q=q, k=k, v=v, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk,
                d=d, scale=float(np.float32(scale)), mask=mask, window=int(window),
                doc_offsets=offsets)


def make_decode(num_seqs: int, Hq: int, Hkv: int, d: int, *, page_size: int = 16,
                len_min: int = 1024, len_max: int = 32768, seed: int = 0,
                seq_lens: list[int] | None = None, max_seq_len: int | None = None,
                tail_fill: str = "zero", extra_pages: int = 0,
                scale: float | None = None) -> dict:
    """Draw one paged-decode problem (bf16 only).

    Context lengths are uniform in [len_min, len_max] unless given.  Every
    sequence's logical pages are laid out in order and then sent to physical
    pages by one seeded permutation of all pages.  Page slots past a
    sequence's length hold zeros (``tail_fill="zero"``) or quiet NaNs
    (``"nan"``); ``extra_pages`` adds that many unreferenced pages filled the
    same way.
    """
    rng = np.random.default_rng(seed)
    if seq_lens is None:
        seq_lens = rng.integers(len_min, len_max + 1, num_seqs).tolist()
    seq_lens = [int(x) for x in seq_lens]
    assert len(seq_lens) == num_seqs
    if max_seq_len is None:
        max_seq_len = max(len_max, max(seq_lens) if seq_lens else 0)
    max_pages = -(-max_seq_len // page_size)
    pages_per_seq = [-(-n // page_size) for n in seq_lens]
    used_pages = int(sum(pages_per_seq))
    num_pages = used_pages + int(extra_pages)
    perm = rng.permutation(num_pages).astype(np.int32)

    block_table = np.full((num_seqs, max(max_pages, 1)), -1, dtype=np.int32)
    g = 0
    for s, npg in enumerate(pages_per_seq):
        block_table[s, :npg] = perm[g:g + npg]
        g += npg

    q = _draw(rng, (num_seqs, Hq, d), "bf16")
    total_tokens = int(sum(seq_lens))
    # physical (page, slot) of every valid token, sequence by sequence
    tok_page = np.empty(total_tokens, dtype=np.int64)
    tok_slot = np.empty(total_tokens, dtype=np.int64)
    t0 = 0
    for s, n in enumerate(seq_lens):
        t = np.arange(n)
        tok_page[t0:t0 + n] = block_table[s, t // page_size]
        tok_slot[t0:t0 + n] = t % page_size
        t0 += n

    fill = np.uint16(0) if tail_fill == "zero" else BF16_QNAN
    pages = []
    for _ in range(2):  # K then V
        vals = _draw(rng, (total_tokens, Hkv, d), "bf16")
        arr = np.full((num_pages, Hkv, page_size, d), fill, dtype=np.uint16)
        arr[tok_page, :, tok_slot, :] = vals
        del vals
        pages.append(arr)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return dict(kind="decode", q=q, k_pages=pages[0], v_pages=pages[1], block_table=block_table,
                seq_lens=np.asarray(seq_lens, dtype=np.int32), num_seqs=num_seqs, Hq=Hq, Hkv=Hkv,
                d=d, page_size=page_size, max_seq_len=int(max_seq_len), scale=float(np.float32(scale)),
                dtype="bf16")


def prefill_config(name: str, seed: int = 0) -> dict:
    c = dict(CONFIGS[name])
    assert c.pop("kind") == "prefill"
    return make_prefill(seed=seed, **c)


def decode_config(name: str, seed: int = 0, **overrides) -> dict:
    c = dict(CONFIGS[name])
    assert c.pop("kind") == "decode"
    c.update(overrides)
    return make_decode(seed=seed, **c)
