"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each test fixes one property that the attention pages or plain mathematics
state, so that a plausible slip in the oracle (a dropped term, a wrong sign
or index, a transposed operand, an off-by-one mask) fails at least one test:

  * brute force in 50-digit arithmetic on tiny inputs, for every mask kind;
  * closed forms: constant V, identical keys, two keys, causal row 0;
  * invariants: probabilities sum to one, key/value permutation;
  * reductions: window >= N is causal, window 1 is the diagonal, the
    document mask is causal attention run per document, GQA is MHA with the
    KV heads repeated, bottom-right causal alignment when Nq < Nk;
  * the worked example printed on the "Attention Is the Bottleneck" page
    (section "FlashAttention: same math, different IO"): the running-max /
    running-sum form agrees with the full softmax to rounding noise;
  * the split-KV log-sum-exp combine of the Flash-Decoding section;
  * the bf16 helpers: widening of every one of the 65,536 bit patterns
    against torch's own conversion and hand-decoded patterns, and rounding
    to the nearest bf16 against torch's float32 rounding and exact ties.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ------------------------------------------------------------ bf16 helpers

def test_from_bf16_bits_every_pattern_matches_torch():
    """All 65,536 bf16 bit patterns widen exactly as torch widens its bfloat16."""
    import torch

    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.from_bf16_bits(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)           # NaNs compared by class
    assert nan.sum() == 2 * 127                          # exponent all ones, mantissa non-zero, both signs
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


@pytest.mark.parametrize("pattern,value", [
    (0x3F80, 1.0), (0xBF80, -1.0), (0xC000, -2.0), (0x3FC0, 1.5), (0x4049, 3.140625),
    (0x0001, 2.0 ** -133),                               # smallest subnormal
    (0x007F, 127 * 2.0 ** -133),                         # largest subnormal
    (0x0080, 2.0 ** -126),                               # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),            # largest finite
    (0x7F80, np.inf), (0xFF80, -np.inf), (0x0000, 0.0),
])
def test_from_bf16_bits_hand_decoded(pattern, value):
    # sign | 8 exponent bits (bias 127) | 7 mantissa bits, decoded by hand above
    got = oracle.from_bf16_bits(np.array([pattern], dtype=np.uint16))[0]
    assert got == value


def test_from_bf16_bits_negative_zero_and_shape():
    got = oracle.from_bf16_bits(np.array([[0x8000, 0x3F80], [0x4000, 0x7FC1]], dtype=np.uint16))
    assert got.shape == (2, 2) and got.dtype == np.float64
    assert got[0, 0] == 0.0 and np.signbit(got[0, 0])
    assert got[0, 1] == 1.0 and got[1, 0] == 2.0 and np.isnan(got[1, 1])


def test_round_to_bf16_matches_torch_on_float32_values():
    """On float32 inputs a single rounding is what torch's float -> bfloat16 does."""
    import torch

    rng = np.random.default_rng(5)
    f = (rng.standard_normal(400_000) * 10.0 ** rng.integers(-44, 38, 400_000)).astype(np.float32)
    f = np.concatenate([f[np.isfinite(f)], np.float32([0.0, -0.0, 1e-45, -3e-39, 3.3e38])])
    ours = oracle.round_to_bf16(f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).double().numpy()
    assert np.array_equal(ours, ref)


def test_round_to_bf16_ties_and_near_ties():
    """Ties go to the even significand; a near-tie that a double rounding
    through float32 would turn into a tie still rounds to the nearer value."""
    u = 2.0 ** -7                                        # spacing in [1, 2)
    cases = [
        (1.0 + u / 2, 1.0),                              # tie, 1.0 is even
        (1.0 + 3 * u / 2, 1.0 + 2 * u),                  # tie, 1 + 2u is even
        (1.0 + u / 2 + 2.0 ** -40, 1.0 + u),             # just above the tie (float32 would drop the 2^-40)
        (1.0 + u / 2 - 2.0 ** -40, 1.0),
        (-(2.0 + u), -2.0),                              # tie at spacing 2u, sign kept
        (2.0 ** -134, 0.0),                              # subnormal tie between 0 and 2^-133
        (3 * 2.0 ** -134, 2.0 ** -132),                  # subnormal tie, even side
        (2.0 ** -134 + 2.0 ** -170, 2.0 ** -133),
        ((2.0 - 2.0 ** -8) * 2.0 ** 127, np.inf),        # halfway to the next binade: overflows
        ((2.0 - 2.0 ** -8) * 2.0 ** 127 * (1 - 2.0 ** -50), (2.0 - 2.0 ** -7) * 2.0 ** 127),
    ]
    x = np.array([c[0] for c in cases])
    want = np.array([c[1] for c in cases])
    assert np.array_equal(oracle.round_to_bf16(x), want)
    assert np.isnan(oracle.round_to_bf16(np.array([np.nan]))[0])


def test_round_to_bf16_is_nearest_and_idempotent():
    """Every result is a bf16 value, no other bf16 value is nearer, and bf16
    values are fixed points."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.from_bf16_bits(bits)
    fin = np.isfinite(vals)
    assert np.array_equal(oracle.round_to_bf16(vals[fin]), vals[fin])
    grid = np.unique(vals[fin])                          # every finite bf16 value, sorted
    x = np.random.default_rng(6).standard_normal(200_000) * 10.0 ** np.random.default_rng(7).integers(-20, 20, 200_000)
    r = oracle.round_to_bf16(x)
    idx = np.searchsorted(grid, x)
    lo, hi = grid[np.clip(idx - 1, 0, grid.size - 1)], grid[np.clip(idx, 0, grid.size - 1)]
    best = np.minimum(np.abs(x - lo), np.abs(x - hi))
    assert np.isin(r, grid).all()
    assert np.array_equal(np.abs(x - r), best)


# ---------------------------------------------------------------- brute force

def _visible_keys(i, Nq, Nk, mask, window, offsets):
    """Visible key set of query row i, enumerated rule by rule."""
    pos = i + Nk - Nq
    if mask == "none":
        return list(range(Nk))
    if mask == "causal":
        return [j for j in range(Nk) if j <= pos]
    if mask == "window":
        return [j for j in range(Nk) if pos - window < j <= pos]
    # document: scan the offsets for the document holding position pos
    if pos < 0:
        return []
    start = None
    for a, b in zip(offsets[:-1], offsets[1:]):
        if a <= pos < b:
            start = a
    return [j for j in range(Nk) if start <= j <= pos]


def _brute(q, k, v, scale, mask, window=0, offsets=None):
    mpmath.mp.dps = 50
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    O = np.zeros(q.shape)
    L = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for i in range(Nq):
                keys = _visible_keys(i, Nq, Nk, mask, window, offsets)
                if not keys:
                    continue
                s = {j: mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[b, h, i, c]) * mpmath.mpf(k[b, hk, j, c])
                                                        for c in range(d)) for j in keys}
                w = {j: mpmath.exp(s[j]) for j in keys}
                tot = mpmath.fsum(w.values())
                for c in range(d):
                    O[b, h, i, c] = float(mpmath.fsum(w[j] * mpmath.mpf(v[b, hk, j, c]) for j in keys) / tot)
                L[b, h, i] = float(mpmath.log(tot))
    return O, L


@pytest.mark.parametrize("mask,window,offsets,Nq,Nk", [
    ("none", 0, None, 5, 6),
    ("causal", 0, None, 6, 6),
    ("causal", 0, None, 3, 6),      # bottom-right alignment, Nq < Nk
    ("causal", 0, None, 6, 4),      # Nq > Nk: the first rows see nothing
    ("window", 1, None, 6, 6),
    ("window", 2, None, 6, 6),
    ("window", 3, None, 4, 6),
    ("document", 0, [0, 2, 5, 6], 6, 6),
    ("document", 0, [0, 1, 6], 6, 6),
])
def test_brute_force_tiny(mask, window, offsets, Nq, Nk):
    B, Hq, Hkv, d = 1, 4, 2, 3
    q, k, v = rnd(1, B, Hq, Nq, d), rnd(2, B, Hkv, Nk, d), rnd(3, B, Hkv, Nk, d)
    scale = 0.7
    o, lse = oracle.attention(q, k, v, scale, mask, window, offsets)
    ob, lb = _brute(q, k, v, scale, mask, window, offsets)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-13)
    assert np.all(o[~fin] == 0.0)


# --------------------------------------------------------------- closed forms

@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 5)])
def test_probabilities_sum_to_one(mask, window):
    # With V the identity matrix, each output row is the probability row itself.
    N = 24
    q, k = rnd(4, 1, 2, N, 8), rnd(5, 1, 2, N, 8)
    v = np.broadcast_to(np.eye(N), (1, 2, N, N)).copy()
    # head dim of V must match q's for the oracle; pad q and k with zeros instead
    qp = np.concatenate([q, np.zeros((1, 2, N, N - 8))], axis=-1)
    kp = np.concatenate([k, np.zeros((1, 2, N, N - 8))], axis=-1)
    p, _ = oracle.attention(qp, kp, v, 0.5, mask, window)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-12)
    assert np.all(p >= 0)
    vis = oracle.visibility(N, N, mask, window)
    assert np.all(p[0, 0][~vis] == 0.0)
    assert np.all(p[0, 0][vis] > 0.0)


@pytest.mark.parametrize("mask,window,offsets", [("none", 0, None), ("causal", 0, None),
                                                 ("window", 3, None), ("document", 0, [0, 7, 9, 20])])
def test_constant_v_gives_constant_output(mask, window, offsets):
    N, d = 20, 6
    c = rnd(6, d)
    v = np.broadcast_to(c, (1, 2, N, d)).copy()
    o, _ = oracle.attention(rnd(7, 1, 4, N, d), rnd(8, 1, 2, N, d), v, 1.3, mask, window, offsets)
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), atol=1e-13)


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 4)])
def test_identical_keys_give_mean_of_visible_values(mask, window):
    N, d, scale = 16, 5, 0.9
    q = rnd(9, 1, 1, N, d)
    kk = rnd(10, d)
    k = np.broadcast_to(kk, (1, 1, N, d)).copy()
    v = rnd(11, 1, 1, N, d)
    o, lse = oracle.attention(q, k, v, scale, mask, window)
    vis = oracle.visibility(N, N, mask, window)
    for i in range(N):
        idx = np.nonzero(vis[i])[0]
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, idx].mean(axis=0), atol=1e-13)
        assert lse[0, 0, i] == pytest.approx(scale * q[0, 0, i] @ kk + math.log(idx.size), abs=1e-13)
    # Q = 0: uniform weights whatever the keys are, LSE = ln(#visible)
    o0, l0 = oracle.attention(np.zeros_like(q), rnd(12, 1, 1, N, d), v, scale, mask, window)
    for i in range(N):
        idx = np.nonzero(vis[i])[0]
        np.testing.assert_allclose(o0[0, 0, i], v[0, 0, idx].mean(axis=0), atol=1e-13)
        assert l0[0, 0, i] == pytest.approx(math.log(idx.size), abs=1e-13)


def test_two_keys_is_a_logistic_blend():
    d, scale = 7, 0.4
    q, k, v = rnd(13, 1, 1, 3, d), rnd(14, 1, 1, 2, d), rnd(15, 1, 1, 2, d)
    o, lse = oracle.attention(q, k, v, scale)
    for i in range(3):
        s0, s1 = scale * q[0, 0, i] @ k[0, 0, 0], scale * q[0, 0, i] @ k[0, 0, 1]
        w = 1.0 / (1.0 + math.exp(-(s0 - s1)))
        np.testing.assert_allclose(o[0, 0, i], w * v[0, 0, 0] + (1 - w) * v[0, 0, 1], atol=1e-13)
        assert lse[0, 0, i] == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), abs=1e-13)


def test_causal_row_zero_copies_first_value():
    q, k, v = rnd(16, 2, 3, 9, 4), rnd(17, 2, 3, 9, 4), rnd(18, 2, 3, 9, 4)
    o, lse = oracle.attention(q, k, v, 0.8, "causal")
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.8 * np.einsum("bhc,bhc->bh", q[:, :, 0], k[:, :, 0]),
                               atol=1e-14)


def test_large_scale_tends_to_hard_max():
    q, k, v = rnd(19, 1, 1, 6, 4), rnd(20, 1, 1, 10, 4), rnd(21, 1, 1, 10, 4)
    o, _ = oracle.attention(q, k, v, 1e3)
    best = np.argmax(q[0, 0] @ k[0, 0].T, axis=1)
    np.testing.assert_allclose(o[0, 0], v[0, 0, best], atol=1e-9)


# ----------------------------------------------------------------- invariants

def test_unmasked_permutation_invariance():
    N, d = 33, 8
    q, k, v = rnd(22, 1, 2, 11, d), rnd(23, 1, 2, N, d), rnd(24, 1, 2, N, d)
    perm = np.random.default_rng(25).permutation(N)
    o1, l1 = oracle.attention(q, k, v, 0.35)
    o2, l2 = oracle.attention(q, k[:, :, perm], v[:, :, perm], 0.35)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)
    # permuting only V must change the output (the pairing of k and v matters)
    o3, _ = oracle.attention(q, k, v[:, :, perm], 0.35)
    assert np.abs(o3 - o1).max() > 1e-3


def test_row_subset_matches_full():
    q, k, v = rnd(26, 1, 2, 40, 8), rnd(27, 1, 2, 40, 8), rnd(28, 1, 2, 40, 8)
    rows = np.array([0, 5, 17, 39])
    of, lf = oracle.attention(q, k, v, 0.3, "causal")
    os_, ls = oracle.attention(q, k, v, 0.3, "causal", rows=rows)
    np.testing.assert_array_equal(os_, of[:, :, rows])
    np.testing.assert_array_equal(ls, lf[:, :, rows])


# ----------------------------------------------------------------- reductions

def test_window_reductions():
    N, d = 30, 6
    q, k, v = rnd(29, 1, 2, N, d), rnd(30, 1, 2, N, d), rnd(31, 1, 2, N, d)
    oc, lc = oracle.attention(q, k, v, 0.5, "causal")
    ow, lw = oracle.attention(q, k, v, 0.5, "window", window=N)
    np.testing.assert_array_equal(ow, oc)
    np.testing.assert_array_equal(lw, lc)
    o1, l1 = oracle.attention(q, k, v, 0.5, "window", window=1)
    assert np.array_equal(o1, v)
    np.testing.assert_allclose(l1, 0.5 * np.einsum("bhnc,bhnc->bhn", q, k), atol=1e-14)


def test_document_mask_is_causal_per_document():
    offsets = [0, 5, 6, 19, 32]
    N, d = 32, 6
    q, k, v = rnd(32, 1, 4, N, d), rnd(33, 1, 2, N, d), rnd(34, 1, 2, N, d)
    o, lse = oracle.attention(q, k, v, 0.6, "document", doc_offsets=offsets)
    for a, b in zip(offsets[:-1], offsets[1:]):
        od, ld = oracle.attention(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], 0.6, "causal")
        np.testing.assert_allclose(o[:, :, a:b], od, atol=1e-13)
        np.testing.assert_allclose(lse[:, :, a:b], ld, atol=1e-13)
    # a single document over everything is the causal mask
    o1, l1 = oracle.attention(q, k, v, 0.6, "document", doc_offsets=[0, N])
    oc, lc = oracle.attention(q, k, v, 0.6, "causal")
    np.testing.assert_array_equal(o1, oc)
    np.testing.assert_array_equal(l1, lc)


def test_gqa_equals_mha_with_repeated_kv_heads():
    Hq, Hkv, N, d = 8, 2, 12, 4
    q, k, v = rnd(35, 2, Hq, N, d), rnd(36, 2, Hkv, N, d), rnd(37, 2, Hkv, N, d)
    o, lse = oracle.attention(q, k, v, 0.5, "causal")
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    om, lm = oracle.attention(q, kr, vr, 0.5, "causal")
    np.testing.assert_array_equal(o, om)
    np.testing.assert_array_equal(lse, lm)
    # the interleaved grouping (kv head = q head % Hkv) is a different result
    ki, vi = np.tile(k, (1, Hq // Hkv, 1, 1)), np.tile(v, (1, Hq // Hkv, 1, 1))
    oi, _ = oracle.attention(q, ki, vi, 0.5, "causal")
    assert np.abs(oi - o).max() > 1e-3


def test_bottom_right_alignment():
    # with Nq < Nk the last query row sees every key, like an unmasked row
    Nq, Nk, d = 4, 10, 5
    q, k, v = rnd(38, 1, 1, Nq, d), rnd(39, 1, 1, Nk, d), rnd(40, 1, 1, Nk, d)
    oc, lc = oracle.attention(q, k, v, 0.7, "causal")
    on, ln = oracle.attention(q, k, v, 0.7, "none")
    np.testing.assert_allclose(oc[:, :, -1], on[:, :, -1], atol=1e-14)
    # and row i sees exactly the first i + 1 + (Nk - Nq) keys
    for i in range(Nq):
        n = i + 1 + Nk - Nq
        oi, li = oracle.attention(q[:, :, i:i + 1], k[:, :, :n], v[:, :, :n], 0.7, "none")
        np.testing.assert_allclose(oc[:, :, i], oi[:, :, 0], atol=1e-14)
        np.testing.assert_allclose(lc[:, :, i], li[:, :, 0], atol=1e-14)


def test_rows_that_see_nothing():
    Nq, Nk = 6, 3
    q, k, v = rnd(41, 1, 1, Nq, 4), rnd(42, 1, 1, Nk, 4), rnd(43, 1, 1, Nk, 4)
    o, lse = oracle.attention(q, k, v, 1.0, "causal")
    assert np.all(o[0, 0, :3] == 0) and np.all(np.isneginf(lse[0, 0, :3]))
    assert np.all(np.isfinite(lse[0, 0, 3:]))
    o, lse = oracle.attention(q, k[:, :, :0], v[:, :, :0], 1.0, "none")
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ------------------------------------------------ the page's worked example

def _online_softmax_one_query(q, K, V, block):
    """Running max / running sum over key blocks, written out for one query."""
    scale = 1.0 / math.sqrt(q.shape[0])
    run_max, run_sum = -math.inf, 0.0
    acc = np.zeros(V.shape[1])
    for a in range(0, K.shape[0], block):
        s = (K[a:a + block] @ q) * scale
        new_max = max(run_max, float(s.max()))
        shrink = math.exp(run_max - new_max)          # 0 on the first block
        w = np.exp(s - new_max)
        run_sum = run_sum * shrink + w.sum()
        acc = acc * shrink + w @ V[a:a + block]
        run_max = new_max
    return acc / run_sum


def test_worked_example_online_softmax_matches_oracle():
    g = json.load(open(os.path.join(GOLDEN, "online_softmax_worked_example.json")))
    rng = np.random.default_rng(g["seed"])
    q = rng.standard_normal(g["d"])
    K = rng.standard_normal((g["n_keys"], g["d"]))
    V = rng.standard_normal((g["n_keys"], g["d"]))
    tiled = _online_softmax_one_query(q, K, V, g["block"])
    o, _ = oracle.attention(q[None, None, None, :], K[None, None], V[None, None], 1.0 / math.sqrt(g["d"]))
    diff = np.abs(o[0, 0, 0] - tiled).max()
    assert diff < 100 * g["printed_max_abs_diff"]
    # and every block size, including ragged tails, gives the same answer
    for block in (1, 7, 64, 1000, 4096):
        assert np.abs(_online_softmax_one_query(q, K, V, block) - o[0, 0, 0]).max() < 1e-14


# ------------------------------------------------ split-KV log-sum-exp combine

def test_split_lse_combine_equals_whole():
    N, d = 100, 8
    q, k, v = rnd(44, 1, 3, 1, d), rnd(45, 1, 3, N, d), rnd(46, 1, 3, N, d)
    o, lse = oracle.attention(q, k, v, 0.4)
    cuts = [0, 13, 14, 50, 99, 100]
    parts = [oracle.attention(q, k[:, :, a:b], v[:, :, a:b], 0.4) for a, b in zip(cuts[:-1], cuts[1:])]
    L = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    O = sum(np.exp(p[1] - L)[..., None] * p[0] for p in parts)
    np.testing.assert_allclose(L, lse, atol=1e-14)
    np.testing.assert_allclose(O, o, atol=1e-14)


# ---------------------------------------------------------------- paged decode

def test_paged_decode_equals_contiguous_attention():
    S, Hq, Hkv, d, P = 3, 4, 2, 8, 16
    lens = [1, 37, 64]
    rng = np.random.default_rng(47)
    q = rng.standard_normal((S, Hq, d))
    conts = [(rng.standard_normal((Hkv, n, d)), rng.standard_normal((Hkv, n, d))) for n in lens]
    npages = sum(-(-n // P) for n in lens)
    perm = rng.permutation(npages)
    kp = np.full((npages, Hkv, P, d), np.nan)
    vp = np.full((npages, Hkv, P, d), np.nan)
    bt = np.full((S, 4), -1, dtype=np.int32)
    g = 0
    for s, n in enumerate(lens):
        for p in range(-(-n // P)):
            phys = perm[g]
            g += 1
            bt[s, p] = phys
            m = min(P, n - p * P)
            kp[phys, :, :m] = conts[s][0][:, p * P:p * P + m]
            vp[phys, :, :m] = conts[s][1][:, p * P:p * P + m]
    o, lse = oracle.paged_decode(q, kp, vp, bt, np.array(lens), 0.3)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))   # NaN tails never read
    for s, n in enumerate(lens):
        oc, lc = oracle.attention(q[s][None, :, None, :], conts[s][0][None], conts[s][1][None], 0.3)
        np.testing.assert_allclose(o[s], oc[0, :, 0], atol=1e-14)
        np.testing.assert_allclose(lse[s], lc[0, :, 0], atol=1e-14)


def test_generated_decode_layout_matches_oracle_gather():
    c = workloads.make_decode(4, 8, 2, 16, len_min=5, len_max=70, seed=3, tail_fill="nan")
    o, lse = oracle.paged_decode(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                 c["scale"], dtype="bf16")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


# ------------------------------------------------ chunked prefill over pages

def _build_paged(conts, P, rng, fill=np.nan):
    """Page the contiguous [Hkv, n, d] K/V of each sequence through one random permutation."""
    lens = [c[0].shape[1] for c in conts]
    Hkv, d = conts[0][0].shape[0], conts[0][0].shape[2]
    npages = max(1, sum(-(-n // P) for n in lens))
    perm = rng.permutation(npages)
    kp = np.full((npages, Hkv, P, d), fill)
    vp = np.full((npages, Hkv, P, d), fill)
    bt = np.full((len(lens), max(1, max(-(-n // P) for n in lens))), -1, dtype=np.int32)
    g = 0
    for s, n in enumerate(lens):
        for p in range(-(-n // P)):
            phys = perm[g]
            g += 1
            bt[s, p] = phys
            m = min(P, n - p * P)
            kp[phys, :, :m] = conts[s][0][:, p * P:p * P + m]
            vp[phys, :, :m] = conts[s][1][:, p * P:p * P + m]
    return kp, vp, bt


def _brute_paged_prefill(q, kp, vp, bt, lens, offs, scale, mask, window):
    """50-digit reference read token by token through the block table (no gather)."""
    mpmath.mp.dps = 50
    T, Hq, d = q.shape
    Hkv, P = kp.shape[1], kp.shape[2]
    g = Hq // Hkv
    O = np.zeros(q.shape)
    L = np.full((T, Hq), -np.inf)
    for s in range(len(lens)):
        n, Ls = offs[s + 1] - offs[s], lens[s]
        for i in range(n):
            keys = _visible_keys(i, n, Ls, mask, window, None)
            for h in range(Hq):
                if not keys:
                    continue
                hk = h // g
                kv = {j: (kp[bt[s, j // P], hk, j % P], vp[bt[s, j // P], hk, j % P]) for j in keys}
                sc = {j: mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[offs[s] + i, h, c]) * mpmath.mpf(kv[j][0][c])
                                                         for c in range(d)) for j in keys}
                w = {j: mpmath.exp(sc[j]) for j in keys}
                tot = mpmath.fsum(w.values())
                for c in range(d):
                    O[offs[s] + i, h, c] = float(mpmath.fsum(w[j] * mpmath.mpf(kv[j][1][c]) for j in keys) / tot)
                L[offs[s] + i, h] = float(mpmath.log(tot))
    return O, L


@pytest.mark.parametrize("mask,window", [("causal", 0), ("none", 0), ("window", 4)])
def test_paged_prefill_brute_force_tiny(mask, window):
    # chunk < context, chunk = context, a single new token, and a chunk longer
    # than an empty context (its rows see nothing)
    Hq, Hkv, d, P = 4, 2, 3, 16
    lens, chunks = [20, 5, 33, 0], [3, 5, 1, 2]
    rng = np.random.default_rng(61)
    conts = [(rng.standard_normal((Hkv, n, d)), rng.standard_normal((Hkv, n, d))) for n in lens]
    kp, vp, bt = _build_paged(conts, P, rng)
    offs = np.concatenate([[0], np.cumsum(chunks)])
    q = rng.standard_normal((offs[-1], Hq, d))
    o, lse = oracle.paged_prefill(q, kp, vp, bt, np.array(lens), offs, 0.6, mask, window)
    ob, lb = _brute_paged_prefill(q, kp, vp, bt, lens, offs, 0.6, mask, window)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-13)
    assert np.all(o[~fin] == 0.0)
    assert not fin[offs[3]:].any()     # empty context: no key for any row


def test_paged_prefill_single_token_chunks_equal_decode():
    c = workloads.make_decode(5, 8, 2, 16, len_min=3, len_max=90, seed=8, tail_fill="nan")
    offs = np.arange(6)
    od, ld = oracle.paged_decode(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                 c["scale"], dtype="bf16")
    op, lp = oracle.paged_prefill(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"], offs,
                                  c["scale"], "causal", dtype="bf16")
    np.testing.assert_array_equal(op, od)
    np.testing.assert_array_equal(lp, ld)


def test_paged_prefill_ignores_page_placement():
    Hq, Hkv, d, P = 4, 1, 5, 16
    lens, chunks = [40, 17], [12, 17]
    rng = np.random.default_rng(5)
    conts = [(rng.standard_normal((Hkv, n, d)), rng.standard_normal((Hkv, n, d))) for n in lens]
    offs = np.concatenate([[0], np.cumsum(chunks)])
    q = rng.standard_normal((offs[-1], Hq, d))
    res = []
    for seed in (1, 2):
        kp, vp, bt = _build_paged(conts, P, np.random.default_rng(seed))
        res.append(oracle.paged_prefill(q, kp, vp, bt, np.array(lens), offs, 0.4))
    np.testing.assert_allclose(res[0][0], res[1][0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(res[0][1], res[1][1], rtol=0, atol=1e-15)


def test_generated_chunked_layout_is_nan_safe():
    c = workloads.make_chunked_prefill(3, 4, 2, 16, prefix_min=0, prefix_max=40, chunk_min=1, chunk_max=30,
                                       seed=4, tail_fill="nan")
    o, lse = oracle.paged_prefill(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                  c["q_offsets"], c["scale"], "causal", dtype="bf16")
    assert o.shape == (int(c["q_offsets"][-1]), 4, 16)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


# ------------------------------------------------------------------- sinks

def _brute_sinks(q, k, v, scale, mask, window, sink_tokens, sinks):
    """50-digit reference: visible keys by rule (window plus the first sink_tokens
    keys, causally), and a per-head sink term e^sink in every denominator."""
    mpmath.mp.dps = 50
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    g = Hq // Hkv
    O = np.zeros(q.shape)
    L = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for i in range(Nq):
                pos = i + Nk - Nq
                keys = _visible_keys(i, Nq, Nk, mask, window, None)
                if mask == "window":
                    keys = sorted(set(keys) | {j for j in range(min(sink_tokens, Nk)) if j <= pos})
                w = {j: mpmath.exp(mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[b, h, i, c]) * mpmath.mpf(k[b, hk, j, c])
                                                                   for c in range(d))) for j in keys}
                tot = mpmath.fsum(w.values())
                if sinks is not None:
                    tot += mpmath.exp(mpmath.mpf(sinks[h]))
                if tot == 0:
                    continue
                for c in range(d):
                    O[b, h, i, c] = float(mpmath.fsum(w[j] * mpmath.mpf(v[b, hk, j, c]) for j in keys) / tot)
                L[b, h, i] = float(mpmath.log(tot))
    return O, L


@pytest.mark.parametrize("mask,window,sink_tokens,with_logits", [
    ("window", 2, 2, False), ("window", 3, 1, True), ("window", 2, 9, False),
    ("causal", 0, 0, True), ("none", 0, 0, True), ("window", 1, 0, True),
])
def test_sinks_brute_force_tiny(mask, window, sink_tokens, with_logits):
    B, Hq, Hkv, d, Nq, Nk = 1, 4, 2, 3, 7, 8
    q, k, v = rnd(71, B, Hq, Nq, d), rnd(72, B, Hkv, Nk, d), rnd(73, B, Hkv, Nk, d)
    sinks = np.array([0.3, -1.2, 2.5, -40.0]) if with_logits else None
    o, lse = oracle.attention(q, k, v, 0.8, mask, window, sink_tokens=sink_tokens, sink_logits=sinks)
    ob, lb = _brute_sinks(q, k, v, 0.8, mask, window, sink_tokens, sinks)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-13)


def test_sink_logit_is_one_more_denominator_term():
    # with sink σ: LSE' = logaddexp(LSE, σ) and O' = O · exp(LSE − LSE'); rows
    # that see nothing get O = 0, LSE = σ
    q, k, v = rnd(81, 1, 4, 9, 8), rnd(82, 1, 2, 6, 8), rnd(83, 1, 2, 6, 8)
    sinks = np.array([-3.0, 0.0, 1.5, 6.0])
    o, lse = oracle.attention(q, k, v, 0.5, "causal")          # Nq > Nk: rows 0..2 see nothing
    os_, ls_ = oracle.attention(q, k, v, 0.5, "causal", sink_logits=sinks)
    want_l = np.logaddexp(lse, sinks[None, :, None])
    np.testing.assert_allclose(ls_, want_l, rtol=0, atol=1e-13)
    fin = np.isfinite(lse)
    scale_o = np.where(fin, np.exp(np.where(fin, lse, 0.0) - want_l), 0.0)
    np.testing.assert_allclose(os_, o * scale_o[..., None], rtol=0, atol=1e-13)
    assert np.all(os_[~fin] == 0.0) and np.allclose(ls_[~fin], np.broadcast_to(sinks[None, :, None], ls_.shape)[~fin])


def test_sink_reductions():
    q, k, v = rnd(91, 1, 2, 12, 4), rnd(92, 1, 2, 12, 4), rnd(93, 1, 2, 12, 4)
    base = oracle.attention(q, k, v, 0.9, "window", 3)
    # no sink tokens = the plain window; a -inf sink logit = no sink
    for got in (oracle.attention(q, k, v, 0.9, "window", 3, sink_tokens=0),
                oracle.attention(q, k, v, 0.9, "window", 3, sink_logits=np.full(2, -np.inf))):
        np.testing.assert_array_equal(got[0], base[0])
        np.testing.assert_array_equal(got[1], base[1])
    # sink tokens covering every key = causal
    c = oracle.attention(q, k, v, 0.9, "causal")
    w = oracle.attention(q, k, v, 0.9, "window", 3, sink_tokens=12)
    np.testing.assert_allclose(w[0], c[0], atol=1e-15)
    np.testing.assert_allclose(w[1], c[1], atol=1e-15)
    # and a visibility check of the rule itself: key 0 stays visible from every row
    vis = oracle.visibility(12, 12, "window", 3, sink_tokens=1)
    assert vis[:, 0].all() and vis.sum() == sum(min(3, i + 1) + (1 if i >= 3 else 0) for i in range(12))
    with pytest.raises(ValueError):
        oracle.visibility(4, 4, "causal", sink_tokens=1)


def test_paged_paths_carry_the_sink():
    c = workloads.make_decode(3, 4, 2, 8, len_min=0, len_max=40, seq_lens=[0, 17, 33], max_seq_len=40, seed=9,
                              tail_fill="nan")
    sinks = np.array([0.5, -1.0, 2.0, 0.0])
    o, lse = oracle.paged_decode(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"], c["scale"],
                                 dtype="bf16", sink_logits=sinks)
    assert np.all(o[0] == 0.0) and np.array_equal(lse[0], sinks)          # empty cache: LSE = sink
    op, lp = oracle.paged_prefill(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                  np.arange(4), c["scale"], "causal", dtype="bf16", sink_logits=sinks)
    np.testing.assert_array_equal(op, o)
    np.testing.assert_array_equal(lp, lse)


# ---------------------------------------------------------------- backward

def _loss(q, k, v, do, scale, mask, window, offsets, sink_tokens, sinks):
    o, _ = oracle.attention(q, k, v, scale, mask, window, offsets, sink_tokens=sink_tokens, sink_logits=sinks)
    return float(np.sum(o * do))


@pytest.mark.parametrize("mask,window,offsets,Nq,Nk,sink_tokens,with_sinks", [
    ("none", 0, None, 5, 6, 0, False), ("causal", 0, None, 6, 6, 0, False), ("causal", 0, None, 7, 5, 0, True),
    ("window", 2, None, 6, 6, 1, True), ("document", 0, [0, 2, 5, 6], 6, 6, 0, False),
])
def test_backward_matches_central_differences(mask, window, offsets, Nq, Nk, sink_tokens, with_sinks):
    B, Hq, Hkv, d = 1, 4, 2, 3
    q, k, v = rnd(101, B, Hq, Nq, d), rnd(102, B, Hkv, Nk, d), rnd(103, B, Hkv, Nk, d)
    do = rnd(104, B, Hq, Nq, d)
    sinks = np.array([0.4, -0.8, 1.1, 0.0]) if with_sinks else None
    scale = 0.7
    dq, dk, dv, ds = oracle.attention_backward(q, k, v, do, scale, mask, window, offsets, sink_tokens, sinks)
    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h
            lp = _loss(q, k, v, do, scale, mask, window, offsets, sink_tokens, sinks)
            arr[idx] = old - h
            lm = _loss(q, k, v, do, scale, mask, window, offsets, sink_tokens, sinks)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=0, atol=1e-7, err_msg=name)
    if with_sinks:
        for hh in range(Hq):
            sp, sm = sinks.copy(), sinks.copy()
            sp[hh] += h
            sm[hh] -= h
            num = (_loss(q, k, v, do, scale, mask, window, offsets, sink_tokens, sp)
                   - _loss(q, k, v, do, scale, mask, window, offsets, sink_tokens, sm)) / (2 * h)
            assert abs(ds[hh] - num) < 1e-7
    else:
        assert ds is None


@pytest.mark.parametrize("mask,window", [("causal", 0), ("window", 9), ("none", 0)])
def test_backward_matches_torch_autograd(mask, window):
    # an independent forward written in torch (explicit masked softmax),
    # differentiated by autograd in float64
    import torch
    B, Hq, Hkv, N, d = 2, 4, 2, 40, 16
    q, k, v, do = rnd(111, B, Hq, N, d), rnd(112, B, Hkv, N, d), rnd(113, B, Hkv, N, d), rnd(114, B, Hq, N, d)
    sinks = np.array([0.2, 1.5, -0.7, 3.0])
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ts = torch.tensor(sinks, requires_grad=True)
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    allowed = torch.ones(N, N, dtype=torch.bool) if mask == "none" else (j <= i)
    if mask == "window":
        allowed = allowed & (i - j < window)
    kk = tk.repeat_interleave(Hq // Hkv, dim=1)
    vv = tv.repeat_interleave(Hq // Hkv, dim=1)
    s = 0.3 * tq @ kk.transpose(-1, -2)
    s = s.masked_fill(~allowed, float("-inf"))
    s = torch.cat([s, ts[None, :, None, None].expand(B, Hq, N, 1)], dim=-1)
    p = torch.softmax(s, dim=-1)[..., :N]
    (p @ vv * torch.tensor(do)).sum().backward()
    dq, dk, dv, ds = oracle.attention_backward(q, k, v, do, 0.3, mask, window, sink_logits=sinks)
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad), (ds, ts.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=0, atol=1e-12)


def test_backward_key_shift_invariance_and_sink_sum():
    # adding one vector to every visible key of a row shifts all its scores
    # equally, which softmax ignores: without a sink the key gradients sum to
    # zero; with a sink that sum is scale · Σ_i (Σ_j dS_ij) q_i, and
    # Σ_ij dS_ij = -dsink (per head, no GQA here)
    q, k, v, do = rnd(121, 1, 2, 12, 5), rnd(122, 1, 2, 12, 5), rnd(123, 1, 2, 12, 5), rnd(124, 1, 2, 12, 5)
    _, dk, _, _ = oracle.attention_backward(q, k, v, do, 0.5, "causal")
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    sinks = np.array([0.5, -1.0])
    _, dk_s, _, ds = oracle.attention_backward(q, k, v, do, 0.5, "none", sink_logits=sinks)
    # with a sink, row i's key scores sum their gradient to Σ_j dS_ij =
    # Σ_j P_ij dP_ij - D_i (1 - P_sink,i) = P_sink,i D_i, so
    # Σ_j dK_j = scale Σ_i P_sink,i D_i q_i, while dsink = -Σ_i P_sink,i D_i
    o, lse = oracle.attention(q, k, v, 0.5, "none", sink_logits=sinks)
    D = np.sum(do * o, axis=-1)                                  # [1, H, N]
    psink = np.exp(sinks[None, :, None] - lse)                   # [1, H, N]
    want = 0.5 * np.einsum("bhn,bhnd->bhd", psink * D, q)
    np.testing.assert_allclose(dk_s.sum(axis=2), want, atol=1e-12)
    np.testing.assert_allclose(ds, -np.sum(psink * D, axis=(0, 2)), atol=1e-12)


def test_backward_rows_that_see_nothing():
    q, k, v, do = rnd(131, 1, 2, 8, 4), rnd(132, 1, 2, 5, 4), rnd(133, 1, 2, 5, 4), rnd(134, 1, 2, 8, 4)
    dq, dk, dv, _ = oracle.attention_backward(q, k, v, do, 0.6, "causal")   # rows 0..2 see no key
    assert np.all(dq[:, :, :3] == 0.0)
    assert np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
