"""Plain fp64 CPU oracle for exact attention (prefill), paged decode and
chunked prefill over a paged cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library.

What it computes is the plain definition of softmax attention as the
"Attention Is the Bottleneck" page (samanvya.dev) writes it in "What attention
costs": scores Q·Kᵀ times a scale, a row softmax, then the weighted sum of V.
It follows the three-step textbook structure that page describes in the same
section (scores, then probabilities, then the output), with host memory in the
place of HBM: every row's full score vector is materialised.  There is no
online softmax and no tiling here; the tiled, online form is what the GPU
kernels do, and the pages state that it reaches this same result up to
rounding ("FlashAttention: same math, different IO").

Readings of points the pages leave open (kept identical in the kernels):
  * scale multiplies Q·Kᵀ before the 0 / -inf mask is added; default 1/sqrt(d);
  * LSE is the natural-log log-sum-exp of the scaled visible scores of a row;
  * causal alignment is bottom-right: query i sits at key position i + Nk - Nq;
  * a sliding window of width W lets a query see the W latest keys including
    its own position (the "last W tokens" of the Sliding windows section);
  * the document mask is causal inside each packed document (FlexAttention's
    document masks, "Attention and matrix kernels" page, How it works);
  * grouped-query heads are contiguous groups: kv head = q head // (Hq / Hkv)
    (MQA and GQA section);
  * a row that sees no key has output 0 and LSE -inf (LSE = the sink logit
    when a learned per-head sink is given);
  * sink tokens keep the first keys visible beside a sliding window, and a
    learned per-head sink logit joins each row's softmax denominator with a
    zero value (AIB, Sliding windows and local:global layers);
  * score modifications (FlexAttention's score_mod, "Attention and matrix
    kernels" page, How it works) act on the scaled score of a visible pair
    before the mask: a soft cap c turns it into c·tanh(score / c), then an
    ALiBi-style per-head slope m adds m·(j - pos) with pos = i + Nk - Nq the
    query's key position; the sink logit is not modified.

Parity pins: see tests/test_oracle_pins.py (brute force in 50-digit
arithmetic, closed forms, invariants, reductions and the worked example the
page prints for the online-softmax recurrence).  The two bf16 helpers are
pinned there too: ``from_bf16_bits`` on all 65,536 bit patterns against
torch's own bf16 widening and against hand-decoded patterns, and
``round_to_bf16`` against torch's float32 -> bf16 rounding and against
ties and near-ties that a double rounding through float32 would get wrong.
No function here is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

MASKS = ("none", "causal", "window", "document")


def from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bit patterns (uint16) exactly to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    bf16 keeps 8 significant bits and float32's exponent range.  A finite x
    is m * 2**e with 0.5 <= |m| < 1 (frexp); m * 2**8 is then exact in
    float64 and rint (ties to even) rounds it to the 8-bit significand.  Below
    the smallest normal (2**-126) the spacing stays at 2**-133.  Magnitudes
    from the largest finite bf16 value plus half its spacing up round to
    infinity.  This rounds once, straight from float64: going through float32
    first could round twice.  NaN and infinities pass through.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)                   # below 2**-126 the spacing is fixed at 2**-133
    out = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    big = (2.0 - 2.0 ** -8) * 2.0 ** 127       # halfway between the largest finite value and the next binade
    out = np.where(np.abs(x) >= big, np.copysign(np.inf, x), out)
    return np.where(np.isfinite(x), out, x)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Inputs as the oracle sees them: bf16 bit patterns or float32, widened exactly."""
    if dtype == "bf16":
        return from_bf16_bits(x)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def visibility(Nq: int, Nk: int, mask: str, window: int = 0, doc_offsets=None,
               rows: np.ndarray | None = None, sink_tokens: int = 0) -> np.ndarray:
    """Boolean matrix vis[i, j]: may query row i attend to key j?

    Query i stands at key position pos = i + (Nk - Nq).
      none      every key
      causal    j <= pos
      window    0 <= pos - j < window, or j < sink_tokens and j <= pos (the
                first tokens kept visible beside the recent window, as
                StreamingLLM does: AIB, Sliding windows and local:global layers)
      document  j <= pos and key j lies in the same document as position pos
    """
    if mask not in MASKS:
        raise ValueError(f"unknown mask {mask!r}")
    if sink_tokens and mask != "window":
        raise ValueError("sink tokens apply to the window mask only")
    i = np.arange(Nq) if rows is None else np.asarray(rows)
    pos = (i + (Nk - Nq))[:, None]
    j = np.arange(Nk)[None, :]
    if mask == "none":
        return np.ones((i.size, Nk), dtype=bool)
    if mask == "causal":
        return j <= pos
    if mask == "window":
        if window < 1:
            raise ValueError("window must be >= 1")
        return (pos - j >= 0) & ((pos - j < window) | (j < sink_tokens))
    off = np.asarray(doc_offsets, dtype=np.int64)
    # document id of a key position: the last offset that is <= the position
    doc_of_key = np.searchsorted(off, np.arange(Nk), side="right") - 1
    pos_flat = pos[:, 0]
    doc_of_pos = np.where(pos_flat >= 0,
                          np.searchsorted(off, np.clip(pos_flat, 0, None), side="right") - 1, -1)
    return (j <= pos) & (doc_of_key[None, :] == doc_of_pos[:, None])


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, mask: str = "none",
              window: int = 0, doc_offsets=None, rows=None, row_block: int = 1024,
              sink_tokens: int = 0, sink_logits=None, softcap: float = 0.0, alibi_slopes=None):
    """O = softmax(mod(scale·Q·Kᵀ) + mask)·V and LSE, in float64.

    q [B, Hq, Nq, d], k and v [B, Hkv, Nk, d] (float64).  Returns o with q's
    shape (or [B, Hq, len(rows), d] when ``rows`` selects query rows) and
    lse [B, Hq, Nq] (or [B, Hq, len(rows)]).  Rows are independent, so a row
    subset is exact for the rows it lists.

    ``sink_logits`` [Hq] (optional): a learned sink per query head, as gpt-oss
    has (AIB, Sliding windows and local:global layers): each row's softmax
    runs over its visible scores plus one more entry whose logit is the
    head's sink and whose value is zero.  It only enlarges the denominator:
    O = Σ e^s v / (Σ e^s + e^sink), LSE = ln(Σ e^s + e^sink); a row with no
    visible key gets O = 0 and LSE = sink.  ``sink_tokens``: see visibility.

    ``softcap`` > 0 and ``alibi_slopes`` [Hq] (optional) are the score
    modifications: score -> softcap·tanh(score / softcap), then
    score + slope[h]·(j - pos_i), pos_i = i + Nk - Nq.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    row_idx = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = row_idx.size
    sinks = None if sink_logits is None else np.asarray(sink_logits, dtype=np.float64).reshape(Hq)
    slopes = None if alibi_slopes is None else np.asarray(alibi_slopes, dtype=np.float64).reshape(Hq)
    softcap = float(softcap)
    if softcap < 0 or not np.isfinite(softcap):
        raise ValueError("softcap must be finite and >= 0")
    o = np.zeros((B, Hq, R, d), dtype=np.float64)
    lse = np.full((B, Hq, R), -np.inf, dtype=np.float64)
    if sinks is not None:
        lse[:] = sinks[None, :, None]          # the rows that see no key keep LSE = sink
    if R == 0 or Nk == 0:
        return o, lse
    scale = float(scale)
    for r0 in range(0, R, row_block):
        sel = row_idx[r0:r0 + row_block]
        vis = visibility(Nq, Nk, mask, window, doc_offsets, rows=sel, sink_tokens=sink_tokens)
        any_vis = vis.any(axis=1)
        for b in range(B):
            for h in range(Hq):
                hk = h // group
                # step 1: scores for the full rows, their modifications, then the additive mask
                s = scale * (q[b, h, sel, :] @ k[b, hk].T)
                if softcap > 0:
                    s = softcap * np.tanh(s / softcap)
                if slopes is not None:         # key position minus the query's key position
                    s = s + slopes[h] * (np.arange(Nk)[None, :] - (sel + Nk - Nq)[:, None])
                s = np.where(vis, s, -np.inf)
                if sinks is not None:          # the sink joins each row as one more score
                    s = np.concatenate([s, np.full((sel.size, 1), sinks[h])], axis=1)
                # step 2: probabilities
                m = np.max(s, axis=1, keepdims=True)
                m = np.where(np.isfinite(m), m, 0.0)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                safe_l = np.where(l > 0, l, 1.0)
                p = e / safe_l
                # step 3: output (the sink's value is zero) and the log-sum-exp statistic
                o[b, h, r0:r0 + sel.size] = p[:, :Nk] @ v[b, hk]
                lse_blk = m[:, 0] + np.log(safe_l[:, 0])
                if sinks is None:
                    lse[b, h, r0:r0 + sel.size] = np.where(any_vis, lse_blk, -np.inf)
                else:
                    lse[b, h, r0:r0 + sel.size] = lse_blk
        o[:, :, r0:r0 + sel.size][:, :, ~any_vis] = 0.0
    return o, lse


def gather_sequence(pages: np.ndarray, block_table_row: np.ndarray, seq_len: int) -> np.ndarray:
    """Contiguous [Hkv, seq_len, d] view of one sequence's paged K or V.

    pages [num_pages, Hkv, page_size, d]; logical token t lives in physical
    page block_table_row[t // page_size], slot t % page_size.
    """
    page_size = pages.shape[2]
    t = np.arange(seq_len)
    phys = np.asarray(block_table_row)[t // page_size]
    return np.transpose(pages[phys, :, t % page_size, :], (1, 0, 2))


def paged_decode(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray, block_table: np.ndarray,
                 seq_lens: np.ndarray, scale: float, seqs=None, dtype: str = "f64", sink_logits=None,
                 softcap: float = 0.0, alibi_slopes=None):
    """One-token decode over a paged KV cache, in float64.

    q [S, Hq, d]; k_pages/v_pages [P, Hkv, page_size, d]; block_table
    [S, max_pages]; seq_lens [S].  The single query of a sequence is its
    newest token, so it sees every one of the sequence's ``seq_len`` cached
    keys (so with the score modifications it sits at position seq_len - 1).
    Returns o [S', Hq, d], lse [S', Hq] for the sequences ``seqs``
    (default: all).  With ``dtype="bf16"`` q and the pages are raw bf16 bit
    patterns, widened here one gathered sequence at a time.
    """
    q = to_f64(q, dtype) if dtype == "bf16" else np.asarray(q, dtype=np.float64)
    S, Hq, d = q.shape
    seqs = range(S) if seqs is None else list(seqs)
    out_o = np.zeros((len(seqs), Hq, d), dtype=np.float64)
    out_l = np.full((len(seqs), Hq), -np.inf, dtype=np.float64)
    if sink_logits is not None:
        out_l[:] = np.asarray(sink_logits, dtype=np.float64)[None, :]
    for n, s in enumerate(seqs):
        L = int(seq_lens[s])
        if L == 0:
            continue
        ks = gather_sequence(k_pages, block_table[s], L)
        vs = gather_sequence(v_pages, block_table[s], L)
        if dtype == "bf16":
            ks, vs = from_bf16_bits(ks), from_bf16_bits(vs)
        else:
            ks, vs = ks.astype(np.float64), vs.astype(np.float64)
        o, lse = attention(q[s][None, :, None, :], ks[None], vs[None], scale, "none", sink_logits=sink_logits,
                           softcap=softcap, alibi_slopes=alibi_slopes)
        out_o[n] = o[0, :, 0, :]
        out_l[n] = lse[0, :, 0]
    return out_o, out_l


def paged_prefill(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray, block_table: np.ndarray,
                  seq_lens: np.ndarray, q_offsets: np.ndarray, scale: float, mask: str = "causal",
                  window: int = 0, seqs=None, dtype: str = "f64", sink_tokens: int = 0, sink_logits=None,
                  softcap: float = 0.0, alibi_slopes=None):
    """Chunked prefill over a paged KV cache, in float64.

    The serving pattern that pairs a tiled attention kernel with KV paging
    (the FlashAttention serving-value question page, Real-world examples;
    paged kernels, "Attention and matrix kernels" page).  Sequence s holds
    seq_lens[s] cached tokens, the newest Nq_s = q_offsets[s+1] - q_offsets[s]
    of which are the chunk being prefilled; its queries are the token-major
    rows q[q_offsets[s]:q_offsets[s+1]] of q [total_q, Hq, d].  Query i of a
    chunk sits at key position i + seq_len - Nq_s (bottom-right alignment),
    so under the causal mask it sees keys 0 .. i + seq_len - Nq_s.

    Each sequence's K and V are gathered through its block table into
    contiguous arrays and handed to ``attention`` with Nq = Nq_s, Nk =
    seq_len.  Returns o [total_q', Hq, d] and lse [total_q', Hq] for the
    tokens of the sequences ``seqs`` (default: all), in their order.
    ``dtype="bf16"``: q and the pages are raw bf16 bit patterns.
    """
    q = to_f64(q, dtype) if dtype == "bf16" else np.asarray(q, dtype=np.float64)
    T, Hq, d = q.shape
    offs = np.asarray(q_offsets, dtype=np.int64)
    S = offs.size - 1
    seqs = range(S) if seqs is None else list(seqs)
    outs_o, outs_l = [], []
    for s in seqs:
        a, b = int(offs[s]), int(offs[s + 1])
        n, L = b - a, int(seq_lens[s])
        o = np.zeros((n, Hq, d), dtype=np.float64)
        lse = np.full((n, Hq), -np.inf, dtype=np.float64)
        if sink_logits is not None:
            lse[:] = np.asarray(sink_logits, dtype=np.float64)[None, :]
        if n > 0 and L > 0:
            ks = gather_sequence(k_pages, block_table[s], L)
            vs = gather_sequence(v_pages, block_table[s], L)
            if dtype == "bf16":
                ks, vs = from_bf16_bits(ks), from_bf16_bits(vs)
            else:
                ks, vs = ks.astype(np.float64), vs.astype(np.float64)
            qs = np.transpose(q[a:b], (1, 0, 2))[None]          # [1, Hq, n, d]
            os_, ls_ = attention(qs, ks[None], vs[None], scale, mask, window, sink_tokens=sink_tokens,
                                 sink_logits=sink_logits, softcap=softcap, alibi_slopes=alibi_slopes)
            o = np.transpose(os_[0], (1, 0, 2))
            lse = np.transpose(ls_[0], (1, 0))
        outs_o.append(o)
        outs_l.append(lse)
    if not outs_o:
        return np.zeros((0, Hq, d)), np.zeros((0, Hq))
    return np.concatenate(outs_o, axis=0), np.concatenate(outs_l, axis=0)


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, scale: float,
                       mask: str = "none", window: int = 0, doc_offsets=None, sink_tokens: int = 0,
                       sink_logits=None, softcap: float = 0.0, alibi_slopes=None):
    """Gradients of attention, in float64: (dq, dk, dv, dsink).

    The backward pass the "Attention Is the Bottleneck" page describes for
    FlashAttention-2: the forward keeps only O and the per-row log-sum-exp,
    and the backward recomputes the probabilities from them.  Written here
    from the chain rule of the plain definition, with full score rows:
      P  = exp(S - LSE)                    (S = scale Q Kᵀ + mask; the sink,
                                            if any, is inside LSE)
      dV = Pᵀ dO,   dP = dO Vᵀ,   D = rowsum(dO ∘ O) = rowsum(P ∘ dP)
      dS = P ∘ (dP - D),   dQ = scale dS K,   dK = scale dSᵀ Q
      dsink[h] = -Σ_i P_sink,i D_i         (the sink's value is zero)
    q, do [B, Hq, Nq, d]; k, v [B, Hkv, Nk, d].  dk and dv sum over the query
    heads of each KV head's group.  dsink is None without sink logits.

    With the score modifications (see ``attention``) S is the modified score
    and dS its gradient; the chain rule through the cap multiplies it by
    d(c tanh(x / c)) / dx = 1 - tanh²(x / c) before dQ and dK (the slope
    bias does not depend on Q or K).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    group = Hq // Hkv
    sinks = None if sink_logits is None else np.asarray(sink_logits, dtype=np.float64).reshape(Hq)
    slopes = None if alibi_slopes is None else np.asarray(alibi_slopes, dtype=np.float64).reshape(Hq)
    softcap = float(softcap)
    if softcap < 0 or not np.isfinite(softcap):
        raise ValueError("softcap must be finite and >= 0")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsink = None if sinks is None else np.zeros(Hq)
    vis = visibility(Nq, Nk, mask, window, doc_offsets, sink_tokens=sink_tokens)
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            x = scale * (q[b, h] @ k[b, hk].T)
            dx = np.ones_like(x)                       # d(modified score) / dx
            if softcap > 0:
                th = np.tanh(x / softcap)
                x = softcap * th
                dx = 1.0 - th * th
            if slopes is not None:
                x = x + slopes[h] * (np.arange(Nk)[None, :] - (np.arange(Nq) + Nk - Nq)[:, None])
            s = np.where(vis, x, -np.inf)
            cols = [s] if sinks is None else [s, np.full((Nq, 1), sinks[h])]
            full = np.concatenate(cols, axis=1)
            m = np.max(full, axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.exp(full - m)
            l = e.sum(axis=1, keepdims=True)
            p_all = e / np.where(l > 0, l, 1.0)
            p = p_all[:, :Nk]
            o = p @ v[b, hk]
            dP = do[b, h] @ v[b, hk].T
            D = np.sum(do[b, h] * o, axis=1, keepdims=True)
            dS = p * (dP - D) * dx
            dq[b, h] = scale * (dS @ k[b, hk])
            dk[b, hk] += scale * (dS.T @ q[b, h])
            dv[b, hk] += p.T @ do[b, h]
            if sinks is not None:
                dsink[h] -= np.sum(p_all[:, Nk] * D[:, 0])
    return dq, dk, dv, dsink
