"""Pins of the oracle's score modifications (soft cap, ALiBi-style slopes).

The modifications act on each visible pair's scaled score before the mask
(FlexAttention's score_mod, "Attention and matrix kernels" page, How it
works): score -> c·tanh(score / c), then + m_h·(j - pos_i) with
pos_i = i + Nk - Nq.  Each test fixes them by something other than the
oracle's own formula:

  * closed forms: two keys whose scores are c·atanh(a) cap to exactly c·a,
    and zero queries make the ALiBi weights a geometric series;
  * limits: a cap far above the scores leaves plain attention, a cap far
    below them leaves uniform weights over the visible keys;
  * a bound: capped logits lie in [-c, c], so |LSE - ln n_visible| <= c;
  * a reduction: the ALiBi bias is one more head-dim coordinate (m_h / scale
    on the query, the key index on the key), with the query's own constant
    -m_h·pos_i moved into the LSE;
  * brute force in 50-digit arithmetic on tiny inputs, both modifications on,
    for every mask kind.
"""
import math

import mpmath
import numpy as np
import pytest

import oracle
import workloads


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def _two_keys(c, a, scale):
    """q [1,1,1,2], k [1,1,2,2] whose scaled scores are c·atanh(a_j)."""
    x = c * np.arctanh(np.asarray(a, dtype=np.float64))
    q = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    k = np.stack([x / scale, np.zeros(2)], axis=1).reshape(1, 1, 2, 2)
    return q, k


def test_softcap_two_keys_closed_form():
    c, scale = 3.0, 0.7
    a = [0.5, -0.25]
    q, k = _two_keys(c, a, scale)
    v = np.array([[2.0, -1.0], [5.0, 3.0]]).reshape(1, 1, 2, 2)
    o, lse = oracle.attention(q, k, v, scale, softcap=c)
    w = np.exp(c * np.array(a))                   # capped scores are exactly c·a_j
    np.testing.assert_allclose(lse[0, 0, 0], math.log(w.sum()), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[0, 0, 0], (w[:, None] * v[0, 0]).sum(0) / w.sum(), rtol=0, atol=1e-13)


def test_softcap_then_alibi_closed_form():
    # the cap acts first, the bias is added to the capped score: with Nq = 1,
    # Nk = 2 the query sits at position 1, so key j gets m·(j - 1)
    c, scale, m = 2.0, 1.3, 0.75
    a = [0.9, -0.6]
    q, k = _two_keys(c, a, scale)
    v = np.array([[1.0, 0.0], [0.0, 1.0]]).reshape(1, 1, 2, 2)
    o, lse = oracle.attention(q, k, v, scale, "causal", softcap=c, alibi_slopes=[m])
    z = c * np.array(a) + m * (np.arange(2) - 1)
    w = np.exp(z)
    np.testing.assert_allclose(lse[0, 0, 0], math.log(w.sum()), rtol=0, atol=1e-13)
    np.testing.assert_allclose(o[0, 0, 0], w / w.sum(), rtol=0, atol=1e-13)


def test_softcap_limits_and_bound():
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 9, 13, 8
    q, k, v = 3 * rnd(1, B, Hq, Nq, d), 3 * rnd(2, B, Hkv, Nk, d), rnd(3, B, Hkv, Nk, d)
    for mask, window in (("none", 0), ("causal", 0), ("window", 4)):
        plain = oracle.attention(q, k, v, 0.6, mask, window)
        big = oracle.attention(q, k, v, 0.6, mask, window, softcap=1e7)
        np.testing.assert_allclose(big[0], plain[0], rtol=0, atol=1e-9)
        np.testing.assert_allclose(big[1], plain[1], rtol=0, atol=1e-9)
        # c -> 0: every capped logit -> 0, uniform weights over the visible keys
        vis = oracle.visibility(Nq, Nk, mask, window)
        n = vis.sum(1)
        small = oracle.attention(q, k, v, 0.6, mask, window, softcap=1e-9)
        for h in range(Hq):
            mean = (vis.astype(float) @ v[0, h // 2]) / np.maximum(n, 1)[:, None]
            np.testing.assert_allclose(small[0][0, h], mean, rtol=0, atol=1e-8)
            np.testing.assert_allclose(small[1][0, h], np.where(n > 0, np.log(np.maximum(n, 1)), -np.inf),
                                       rtol=0, atol=1e-8)
        # any cap: |LSE - ln n| <= c
        for cap in (0.5, 2.0, 7.0):
            l = oracle.attention(q, k, v, 0.6, mask, window, softcap=cap)[1][0]
            assert np.all(np.abs(l - np.log(n)[None, :]) <= cap + 1e-12)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, 0.6, softcap=-1.0)


def test_alibi_geometric_closed_form():
    # q = 0: scores are all zero, so row i's weights are e^{m (j - pos_i)}
    # over its visible keys j = 0..pos_i (causal): a geometric series
    Nq, Nk, d, m = 5, 8, 4, 0.4
    q = np.zeros((1, 1, Nq, d))
    k, v = rnd(11, 1, 1, Nk, d), rnd(12, 1, 1, Nk, d)
    o, lse = oracle.attention(q, k, v, 0.5, "causal", alibi_slopes=[m])
    r = math.exp(m)
    for i in range(Nq):
        pos = i + Nk - Nq
        tot = (r ** (pos + 1) - 1) / (r - 1) * math.exp(-m * pos)   # sum_{j<=pos} e^{m (j - pos)}
        np.testing.assert_allclose(lse[0, 0, i], math.log(tot), rtol=0, atol=1e-12)
        w = np.array([r ** j for j in range(pos + 1)])
        np.testing.assert_allclose(o[0, 0, i], (w[:, None] * v[0, 0, :pos + 1]).sum(0) / w.sum(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 3)])
def test_alibi_is_one_more_coordinate(mask, window):
    B, Hq, Hkv, Nq, Nk, d, scale = 2, 4, 2, 6, 11, 5, 0.45
    q, k, v = rnd(21, B, Hq, Nq, d), rnd(22, B, Hkv, Nk, d), rnd(23, B, Hkv, Nk, d)
    slopes = np.array([0.5, 0.125, -0.3, 0.0])
    o, lse = oracle.attention(q, k, v, scale, mask, window, alibi_slopes=slopes)
    qe = np.concatenate([q, np.broadcast_to((slopes / scale)[None, :, None, None], (B, Hq, Nq, 1))], axis=3)
    ke = np.concatenate([k, np.broadcast_to(np.arange(Nk, dtype=float)[None, None, :, None], (B, Hkv, Nk, 1))], axis=3)
    ve = np.concatenate([v, np.zeros((B, Hkv, Nk, 1))], axis=3)
    oe, le = oracle.attention(qe, ke, ve, scale, mask, window)
    pos = np.arange(Nq) + Nk - Nq
    np.testing.assert_allclose(o, oe[..., :d], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, le - slopes[None, :, None] * pos[None, None, :], rtol=0, atol=1e-11)


def _brute_mods(q, k, v, scale, mask, window, offsets, cap, slopes):
    mpmath.mp.dps = 50
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    O = np.zeros(q.shape)
    L = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            for i in range(Nq):
                pos = i + Nk - Nq
                if mask == "none":
                    keys = range(Nk)
                elif mask == "causal":
                    keys = [j for j in range(Nk) if j <= pos]
                elif mask == "window":
                    keys = [j for j in range(Nk) if pos - window < j <= pos]
                else:
                    start = max([a for a in offsets[:-1] if a <= pos], default=None) if pos >= 0 else None
                    keys = [] if start is None else [j for j in range(Nk) if start <= j <= pos]
                z = {}
                for j in keys:
                    x = mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[b, h, i, c]) * mpmath.mpf(k[b, h // g, j, c])
                                                        for c in range(d))
                    x = mpmath.mpf(cap) * mpmath.tanh(x / cap)
                    z[j] = x + mpmath.mpf(slopes[h]) * (j - pos)
                if not z:
                    continue
                w = {j: mpmath.exp(z[j]) for j in z}
                tot = mpmath.fsum(w.values())
                for c in range(d):
                    O[b, h, i, c] = float(mpmath.fsum(w[j] * mpmath.mpf(v[b, h // g, j, c]) for j in z) / tot)
                L[b, h, i] = float(mpmath.log(tot))
    return O, L


@pytest.mark.parametrize("mask,window,offsets", [
    ("none", 0, None), ("causal", 0, None), ("window", 2, None), ("document", 0, [0, 3, 4, 8]),
])
def test_score_mods_brute_force_tiny(mask, window, offsets):
    B, Hq, Hkv, d, Nq, Nk = 1, 4, 2, 3, 6, 8
    q, k, v = 2 * rnd(31, B, Hq, Nq, d), 2 * rnd(32, B, Hkv, Nk, d), rnd(33, B, Hkv, Nk, d)
    slopes = np.array([0.25, -0.5, 1.0, 0.0625])
    o, lse = oracle.attention(q, k, v, 0.9, mask, window, doc_offsets=offsets, softcap=1.5, alibi_slopes=slopes)
    ob, lb = _brute_mods(q, k, v, 0.9, mask, window, offsets, 1.5, slopes)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


def test_paged_prefill_carries_the_mods():
    # a single chunk covering the whole cache is plain attention on the gathered sequence
    c = workloads.make_chunked_prefill(2, 4, 2, 8, chunks=[5, 3], prefixes=[7, 0], seed=5, tail_fill="nan")
    slopes = np.array([0.5, -0.25, 0.125, 1.0])
    op, lp = oracle.paged_prefill(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                  c["q_offsets"], c["scale"], "causal", dtype="bf16", softcap=2.0,
                                  alibi_slopes=slopes)
    plain = oracle.paged_prefill(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                 c["q_offsets"], c["scale"], "causal", dtype="bf16")
    assert not np.allclose(op, plain[0])
    offs = c["q_offsets"]
    for s in range(2):
        L = int(c["seq_lens"][s])
        k_seq = oracle.from_bf16_bits(oracle.gather_sequence(c["k_pages"], c["block_table"][s], L))
        v_seq = oracle.from_bf16_bits(oracle.gather_sequence(c["v_pages"], c["block_table"][s], L))
        qs = np.transpose(oracle.to_f64(c["q"], "bf16")[offs[s]:offs[s + 1]], (1, 0, 2))[None]
        o, l = oracle.attention(qs, k_seq[None], v_seq[None], c["scale"], "causal", softcap=2.0, alibi_slopes=slopes)
        np.testing.assert_array_equal(op[offs[s]:offs[s + 1]], np.transpose(o[0], (1, 0, 2)))
        np.testing.assert_array_equal(lp[offs[s]:offs[s + 1]], np.transpose(l[0], (1, 0)))


# ---------------------------------------------------------------- backward

def _mod_loss(q, k, v, do, scale, mask, window, offsets, cap, slopes):
    o, _ = oracle.attention(q, k, v, scale, mask, window, offsets, softcap=cap, alibi_slopes=slopes)
    return float(np.sum(o * do))


@pytest.mark.parametrize("mask,window,offsets,Nq,Nk,cap,with_slopes", [
    ("none", 0, None, 5, 6, 1.2, False), ("causal", 0, None, 6, 6, 0.0, True), ("causal", 0, None, 4, 7, 0.8, True),
    ("window", 2, None, 6, 6, 2.0, True), ("document", 0, [0, 2, 5, 6], 6, 6, 1.5, True),
])
def test_mod_backward_matches_central_differences(mask, window, offsets, Nq, Nk, cap, with_slopes):
    B, Hq, Hkv, d = 1, 4, 2, 3
    q, k, v = 2 * rnd(131, B, Hq, Nq, d), 2 * rnd(132, B, Hkv, Nk, d), rnd(133, B, Hkv, Nk, d)
    do = rnd(134, B, Hq, Nq, d)
    slopes = np.array([0.3, -0.2, 0.7, 0.05]) if with_slopes else None
    scale = 0.9
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, mask, window, offsets, softcap=cap,
                                              alibi_slopes=slopes)
    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _mod_loss(q, k, v, do, scale, mask, window, offsets, cap, slopes)
            arr[idx] = old - h
            lm = _mod_loss(q, k, v, do, scale, mask, window, offsets, cap, slopes)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=0, atol=1e-7, err_msg=name)


def test_mod_backward_matches_torch_autograd():
    # an independent forward in torch (tanh cap, then the bias, then the
    # causal mask), differentiated by autograd in float64
    import torch
    B, Hq, Hkv, Nq, Nk, d, scale, cap = 2, 4, 2, 30, 40, 16, 0.6, 2.5
    q, k, v, do = 2 * rnd(141, B, Hq, Nq, d), 2 * rnd(142, B, Hkv, Nk, d), rnd(143, B, Hkv, Nk, d), rnd(144, B, Hq, Nq, d)
    slopes = np.array([0.5, 0.25, 0.125, 0.0625])
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    pos = torch.arange(Nq)[:, None] + (Nk - Nq)
    j = torch.arange(Nk)[None, :]
    kk = tk.repeat_interleave(Hq // Hkv, dim=1)
    vv = tv.repeat_interleave(Hq // Hkv, dim=1)
    s = cap * torch.tanh(scale * tq @ kk.transpose(-1, -2) / cap)
    s = s + torch.tensor(slopes)[None, :, None, None] * (j - pos).double()
    s = s.masked_fill(~(j <= pos), float("-inf"))
    (torch.softmax(s, dim=-1) @ vv * torch.tensor(do)).sum().backward()
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, scale, "causal", softcap=cap, alibi_slopes=slopes)
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=0, atol=1e-12)


def test_paged_decode_carries_the_mods():
    # one query per sequence at position seq_len - 1: the same as a one-token
    # chunk of the chunked prefill, and for q = 0 the slope bias alone gives
    # the geometric weights e^{m (j - (L - 1))}
    c = workloads.make_decode(3, 4, 2, 8, len_min=0, len_max=40, seq_lens=[0, 17, 33], max_seq_len=40, seed=19,
                              tail_fill="nan")
    slopes = np.array([0.5, -0.25, 0.125, 1.0])
    o, lse = oracle.paged_decode(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"], c["scale"],
                                 dtype="bf16", softcap=1.5, alibi_slopes=slopes)
    op, lp = oracle.paged_prefill(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                  np.arange(4), c["scale"], "causal", dtype="bf16", softcap=1.5, alibi_slopes=slopes)
    np.testing.assert_array_equal(o, op)
    np.testing.assert_array_equal(lse, lp)
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
    zq = np.zeros_like(c["q"])                    # bf16 bit patterns of 0.0
    o0, l0 = oracle.paged_decode(zq, c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"], c["scale"],
                                 dtype="bf16", alibi_slopes=slopes)
    for sq in (1, 2):
        L = int(c["seq_lens"][sq])
        vs = oracle.from_bf16_bits(oracle.gather_sequence(c["v_pages"], c["block_table"][sq], L))
        for h in range(4):
            w = np.exp(slopes[h] * (np.arange(L) - (L - 1)))
            np.testing.assert_allclose(l0[sq, h], math.log(w.sum()), rtol=0, atol=1e-12)
            np.testing.assert_allclose(o0[sq, h], (w[:, None] * vs[h // 2]).sum(0) / w.sum(), rtol=0, atol=1e-12)
