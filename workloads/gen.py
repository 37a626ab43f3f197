"""Seeded generators for the attention workloads.

The structure (document lengths, context lengths, page permutation) is drawn
from ``numpy.random.default_rng(seed)``.  Q, K and V are then float32
standard normals, each tensor from its own stream: draw number n (Q = 1,
K = 2, V = 3) of a problem with seed s is cut into chunks of 2**24 values and
chunk i comes from ``default_rng(SeedSequence([s, n]).spawn(...)[i])``, so
large tensors can be drawn on several threads with a fixed result.  bf16 workloads are rounded to
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

import concurrent.futures as cf
import math
import os

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
    # chunked prefill: each sequence prefills a chunk of new tokens against a
    # cached prefix, all through the paged cache
    "c6_chunked_prefill_16": dict(kind="chunked", num_seqs=16, Hq=32, Hkv=8, d=128, page_size=16,
                                  prefix_min=0, prefix_max=8192, chunk_min=256, chunk_max=2048),
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


CHUNK = 1 << 24


def _draw(seed: int, stream: int, shape, dtype: str):
    """Standard normals for one tensor (see the module docstring for the stream)."""
    n = int(np.prod(shape))
    nchunks = max(1, -(-n // CHUNK))
    kids = np.random.SeedSequence([seed, stream]).spawn(nchunks)
    x = np.empty(n, dtype=np.float32)
    out = np.empty(n, dtype=np.uint16) if dtype == "bf16" else x
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype}")

    def fill(i):
        sl = slice(i * CHUNK, min(n, (i + 1) * CHUNK))
        np.random.default_rng(kids[i]).standard_normal(sl.stop - sl.start, dtype=np.float32, out=x[sl])
        if dtype == "bf16":
            out[sl] = bf16_bits_from_f32(x[sl])

    workers = min(16, len(os.sched_getaffinity(0)), nchunks)
    if workers <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


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
    q = _draw(seed, 1, (B, Hq, Nq, d), dtype)
    k = _draw(seed, 2, (B, Hkv, Nk, d), dtype)
    v = _draw(seed, 3, (B, Hkv, Nk, d), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return dict(kind="prefill", q=q, k=k, v=v, dtype=dtype, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk,
                d=d, scale=float(np.float32(scale)), mask=mask, window=int(window),
                doc_offsets=offsets)


def make_decode(num_seqs: int, Hq: int, Hkv: int, d: int, *, page_size: int = 16,
                len_min: int = 1024, len_max: int = 32768, seed: int = 0,
                seq_lens: list[int] | None = None, max_seq_len: int | None = None,
                tail_fill: str = "zero", extra_pages: int = 0,
                scale: float | None = None, with_values: bool = True) -> dict:
    """Draw one paged-decode problem (bf16 only).

    Context lengths are uniform in [len_min, len_max] unless given.  Every
    sequence's logical pages are laid out in order and then sent to physical
    pages by one seeded permutation of all pages.  K and V values are drawn
    for all slots in physical page order.  Page slots past a
    sequence's length hold zeros (``tail_fill="zero"``) or quiet NaNs
    (``"nan"``); ``extra_pages`` adds that many unreferenced pages filled the
    same way.  ``with_values=False`` stops after the structure (lengths,
    block table) and the query, leaving the page arrays as None.
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

    q = _draw(seed, 1, (num_seqs, Hq, d), "bf16")
    fill = np.uint16(0) if tail_fill == "zero" else BF16_QNAN
    pages = []
    for stream in ((2, 3) if with_values else ()):  # K then V
        # every slot of every page is drawn in physical page order; slots past
        # a sequence's end (and unreferenced pages) are then overwritten
        arr = _draw(seed, stream, (num_pages, Hkv, page_size, d), "bf16")
        for s, n in enumerate(seq_lens):
            if n % page_size:
                arr[block_table[s, n // page_size], :, n % page_size:, :] = fill
        if extra_pages:
            arr[perm[used_pages:]] = fill
        pages.append(arr)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if not with_values:
        pages = [None, None]
    return dict(kind="decode", q=q, k_pages=pages[0], v_pages=pages[1], block_table=block_table,
                seq_lens=np.asarray(seq_lens, dtype=np.int32), num_seqs=num_seqs, Hq=Hq, Hkv=Hkv,
                d=d, page_size=page_size, max_seq_len=int(max_seq_len), scale=float(np.float32(scale)),
                dtype="bf16")


def make_chunked_prefill(num_seqs: int, Hq: int, Hkv: int, d: int, *, page_size: int = 16,
                         prefix_min: int = 0, prefix_max: int = 8192, chunk_min: int = 256,
                         chunk_max: int = 2048, seed: int = 0, chunks: list[int] | None = None,
                         prefixes: list[int] | None = None, tail_fill: str = "zero",
                         extra_pages: int = 0, scale: float | None = None) -> dict:
    """Draw one chunked-prefill problem over a paged cache (bf16 only).

    Sequence s has a cached prefix of prefixes[s] tokens and a chunk of
    chunks[s] new tokens (uniform in [prefix_min, prefix_max] and [chunk_min,
    chunk_max] unless given, drawn from the generator seeded (seed, 6): chunk
    lengths first, then prefixes).  The chunk's own K and V are already in the
    cache, so seq_lens = prefix + chunk; the cache (pages, block table, tail
    fill) is the one make_decode draws for those lengths.  The queries are the
    chunk tokens, token-major q [sum(chunks), Hq, d] (stream 4), with
    q_offsets [num_seqs + 1] the running sums of the chunk lengths.
    """
    rng = np.random.default_rng([seed, 6])
    if chunks is None:
        chunks = rng.integers(chunk_min, chunk_max + 1, num_seqs).tolist()
    if prefixes is None:
        prefixes = rng.integers(prefix_min, prefix_max + 1, num_seqs).tolist()
    chunks = [int(x) for x in chunks]
    prefixes = [int(x) for x in prefixes]
    assert len(chunks) == num_seqs and len(prefixes) == num_seqs
    lens = [a + b for a, b in zip(prefixes, chunks)]
    cache = make_decode(num_seqs, Hq, Hkv, d, page_size=page_size, seed=seed, seq_lens=lens,
                        max_seq_len=max(lens) if lens else 0, tail_fill=tail_fill,
                        extra_pages=extra_pages, scale=scale)
    q_offsets = np.zeros(num_seqs + 1, dtype=np.int32)
    q_offsets[1:] = np.cumsum(chunks)
    q = _draw(seed, 4, (int(q_offsets[-1]), Hq, d), "bf16")
    return dict(kind="chunked", q=q, k_pages=cache["k_pages"], v_pages=cache["v_pages"],
                block_table=cache["block_table"], seq_lens=cache["seq_lens"], q_offsets=q_offsets,
                num_seqs=num_seqs, Hq=Hq, Hkv=Hkv, d=d, page_size=page_size,
                max_seq_len=cache["max_seq_len"], max_q_len=max(chunks) if chunks else 0,
                scale=cache["scale"], dtype="bf16", mask="causal", window=0)


def make_backward(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, *, seed: int = 0, **kw) -> dict:
    """A prefill problem plus the gradient flowing into its output: dO with
    q's shape, standard normal, from stream 5 (bf16 bits like q)."""
    c = make_prefill(B, Hq, Hkv, Nq, Nk, d, seed=seed, **kw)
    c["do"] = _draw(seed, 5, (B, Hq, Nq, d), c["dtype"])
    return c


def prefill_config(name: str, seed: int = 0) -> dict:
    c = dict(CONFIGS[name])
    assert c.pop("kind") == "prefill"
    return make_prefill(seed=seed, **c)


def decode_config(name: str, seed: int = 0, **overrides) -> dict:
    c = dict(CONFIGS[name])
    assert c.pop("kind") == "decode"
    c.update(overrides)
    return make_decode(seed=seed, **c)


def chunked_config(name: str, seed: int = 0, **overrides) -> dict:
    c = dict(CONFIGS[name])
    assert c.pop("kind") == "chunked"
    c.update(overrides)
    return make_chunked_prefill(seed=seed, **c)
