"""Sequences of more than 2^24 keys (d = 128).

A K/V tile's buffer range is the tile's own rows that exist, rows * d * 2
bytes with rows clamped to the tile.  Unclamped, Nk - n0 rows of 256 bytes
wrap 32 bits once Nk - n0 passes 2^24, and the first tile of a sequence of
2^24 + 40 keys would read its rows 40..63 as zeros.

The checks use the closed form the oracle is pinned to for identical keys
(tests/test_oracle_pins.py): with every key zero all scores are equal, so a
row's output is the mean of V over the keys it sees and its LSE is
ln(number of those keys), at any size.  V is zero except a few marked rows
(the first tile's rows 40..63, rows past 2^23 and 2^24, the last rows), each
in a column of its own, so every output column is a count of marked rows the
row sees divided by its key count: a tile read as zeros, or from the wrong
rows, zeroes or moves a column.  These outputs are about 1e-6, so they are
compared relatively: bf16 rounding of the output (2^-9) plus the fp32 sums
(1e-6), bound 2^-8."""
import math

import numpy as np
import pytest
import torch

from exact_io_aware_fwd_amd import attn_fwd
from _gpu_helpers import say

pytestmark = pytest.mark.gpu

D = 128
NK = (1 << 24) + 40
NQ = 128
# marked rows of V: (first row, last row, column, value)
MARKS = [(40, 63, 3, 1.0),                      # the first tile's tail
         ((1 << 23) + 5, (1 << 23) + 70, 17, 2.0),
         ((1 << 24) - 3, (1 << 24) + 30, 64, 4.0),   # across 2^24
         (NK - 10, NK - 1, 127, 8.0)]           # the last rows (seen by the last causal rows only)


def inputs():
    q = torch.randn(1, 4, NQ, D, generator=torch.Generator(device="cuda").manual_seed(5), device="cuda")
    k = torch.zeros(1, 1, NK, D, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(1, 1, NK, D, dtype=torch.bfloat16, device="cuda")
    for a, b, col, val in MARKS:
        v[0, 0, a:b + 1, col] = val
    return q.to(torch.bfloat16), k, v


def expected(last_key: int, first_key: int = 0):
    """Output row and LSE of a query that sees keys first_key..last_key."""
    n = last_key - first_key + 1
    o = np.zeros(D)
    for a, b, col, val in MARKS:
        seen = max(0, min(b, last_key) - max(a, first_key) + 1)
        o[col] += val * seen / n
    return o, math.log(n)


def check(o: torch.Tensor, lse: torch.Tensor, last_keys, label: str, first_keys=None):
    og = o[0].double().cpu().numpy()      # [Hq, NQ, D]
    lg = lse[0].double().cpu().numpy()    # [Hq, NQ]
    worst_rel, worst_lse = 0.0, 0.0
    for i, lk in enumerate(last_keys):
        o_ref, l_ref = expected(lk, 0 if first_keys is None else first_keys[i])
        nz = o_ref != 0
        for h in range(og.shape[0]):
            assert np.all(og[h, i, ~nz] == 0.0), f"{label} row {i}: nonzero output where V is zero"
            rel = np.abs(og[h, i, nz] - o_ref[nz]) / o_ref[nz]
            worst_rel = max(worst_rel, float(rel.max()))
            worst_lse = max(worst_lse, abs(lg[h, i] - l_ref))
    say(f"[long keys] {label}: Nk {NK}, max relative error {worst_rel:.3e}, LSE {worst_lse:.3e}")
    assert worst_rel <= 2.0 ** -8, f"{label}: relative error {worst_rel}"
    assert worst_lse <= 1e-3, f"{label}: LSE error {worst_lse}"


def test_prefill_keys_past_2_24_no_mask():
    q, k, v = inputs()
    o, lse = attn_fwd(q, k, v, scale=1.0 / math.sqrt(D), mask="none")
    torch.cuda.synchronize()
    check(o, lse, [NK - 1] * NQ, "no mask")


def test_prefill_keys_past_2_24_causal_bottom_right():
    q, k, v = inputs()
    o, lse = attn_fwd(q, k, v, scale=1.0 / math.sqrt(D), mask="causal")
    torch.cuda.synchronize()
    check(o, lse, [NK - NQ + i for i in range(NQ)], "causal")


def test_prefill_keys_past_2_24_window_as_wide_as_the_keys():
    """A window of all the keys is the bottom-right causal mask; the window
    mask runs on the 32-key-tile kernel."""
    q, k, v = inputs()
    o, lse = attn_fwd(q, k, v, scale=1.0 / math.sqrt(D), mask="window", window=NK)
    torch.cuda.synchronize()
    check(o, lse, [NK - NQ + i for i in range(NQ)], "window of all keys (32-key tiles)")


def test_prefill_keys_past_2_24_window_edge_through_a_mark():
    """Window 2^23 - 50: row i (position NK - NQ + i) sees keys from
    position - W + 1, an edge that sweeps through the marked rows just past
    2^23 as i grows, inside 32-key tiles whose byte offsets pass 2^31."""
    W = (1 << 23) - 50
    q, k, v = inputs()
    o, lse = attn_fwd(q, k, v, scale=1.0 / math.sqrt(D), mask="window", window=W)
    torch.cuda.synchronize()
    pos = [NK - NQ + i for i in range(NQ)]
    check(o, lse, pos, "window 2^23 - 50 (32-key tiles)", first_keys=[p - W + 1 for p in pos])


def test_backward_rows_past_2_24():
    """The backward's Q and dO tiles over 2^24 + 40 query rows (one 128-key
    tile, no mask).  With every key zero each row's P is 1/128 on every key
    and its O is the mean of V, so (identical-keys closed form, then the
    backward's definitions): dQ = 0; dV_j = sum_i dO_i / 128;
    dK_j = scale / 128 * (sum_i q_i dO_i^T) (v_j - O), with O the bf16 mean of
    V the kernel reads back.  Every query row reaches dV and dK, so a tile read
    short or from the wrong rows moves them.  Bound: the backward tests'
    relative Frobenius error 2e-2; dQ exactly zero."""
    from exact_io_aware_fwd_amd import attn_bwd

    nq, nk = (1 << 24) + 40, 128
    g = torch.Generator(device="cuda").manual_seed(23)
    q = torch.randn(1, 1, nq, D, generator=g, device="cuda").to(torch.bfloat16)
    do = torch.randn(1, 1, nq, D, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.zeros(1, 1, nk, D, dtype=torch.bfloat16, device="cuda")
    v = torch.randn(1, 1, nk, D, generator=g, device="cuda").to(torch.bfloat16)
    o_row = v[0, 0].double().mean(dim=0).to(torch.bfloat16)            # the forward's output of every row
    o = o_row.view(1, 1, 1, D).expand(1, 1, nq, D).contiguous()
    lse = torch.full((1, 1, nq), math.log(nk), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv, _ = attn_bwd(q, k, v, o, do, lse, scale=scale, mask="none")
    torch.cuda.synchronize()

    # references in fp64, a million rows at a time
    col = torch.zeros(D, dtype=torch.float64, device="cuda")
    M = torch.zeros(D, D, dtype=torch.float64, device="cuda")
    for a in range(0, nq, 1 << 20):
        qc, dc = q[0, 0, a:a + (1 << 20)].double(), do[0, 0, a:a + (1 << 20)].double()
        col += dc.sum(dim=0)
        M += qc.T @ dc
    dv_ref = (col / nk).expand(nk, D)
    dk_ref = (scale / nk) * (v[0, 0].double() - o_row.double()) @ M.T

    def rel(x, ref):
        return float(torch.linalg.norm(x[0, 0].double() - ref) / torch.linalg.norm(ref))

    e_dv, e_dk = rel(dv, dv_ref), rel(dk, dk_ref)
    nz = int(torch.count_nonzero(dq))
    say(f"[long rows] backward: Nq {nq}, dV rel-fro {e_dv:.3e}, dK rel-fro {e_dk:.3e}, nonzero dQ {nz}")
    assert nz == 0
    assert e_dv <= 2e-2 and e_dk <= 2e-2
