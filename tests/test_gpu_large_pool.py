"""Page pools larger than 4 GiB.

The chunked prefill and the paged decode build a buffer resource per page
from a 64-bit page address, so a page anywhere in a pool of any size is read
correctly.  Each test copies a small problem's pages past the 4 GiB mark of
a large, otherwise unwritten pool, shifts the block table to match, and
checks the result against the fp64 oracle on the original compact pool."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_io_aware_fwd_amd import attn_paged_decode, attn_paged_prefill
from _gpu_helpers import BF16_TOL, compare, dev, host_f64, say

pytestmark = pytest.mark.gpu

FOUR_GIB = 4 << 30


def far_pool(pages: np.ndarray, extra_bytes: int = FOUR_GIB + (512 << 20)):
    """Device pool whose first `shift` pages are left unwritten and whose
    next pages are `pages`; returns (pool, shift)."""
    page_bytes = int(np.prod(pages.shape[1:])) * 2
    shift = (extra_bytes + page_bytes - 1) // page_bytes
    pool = torch.empty((shift + pages.shape[0],) + tuple(pages.shape[1:]), dtype=torch.bfloat16, device="cuda")
    pool[shift:] = dev(pages, "bf16")
    assert shift * page_bytes > FOUR_GIB
    return pool, shift


def shifted(block_table: np.ndarray, shift: int) -> torch.Tensor:
    bt = np.where(block_table >= 0, block_table + shift, block_table).astype(np.int32)
    return torch.from_numpy(np.ascontiguousarray(bt)).cuda()


def test_chunked_prefill_pages_past_4gib():
    c = workloads.make_chunked_prefill(4, 8, 2, 128, chunks=[70, 1, 200, 33], prefixes=[300, 1500, 0, 64], seed=71,
                                       tail_fill="nan")
    say(f"[case] chunked prefill, pages past 4 GiB: lens={c['seq_lens'].tolist()}")
    kp, shift = far_pool(c["k_pages"])
    vp, _ = far_pool(c["v_pages"])
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    o, lse = attn_paged_prefill(dev(c["q"], "bf16"), kp, vp, shifted(c["block_table"], shift), i32(c["seq_lens"]),
                                i32(c["q_offsets"]), max_seq_len=c["max_seq_len"], max_q_len=c["max_q_len"],
                                scale=c["scale"], mask="causal")
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_prefill(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                        c["q_offsets"], c["scale"], "causal", dtype="bf16")
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, BF16_TOL, "chunked prefill past 4 GiB")
    del kp, vp
    torch.cuda.empty_cache()


def test_paged_decode_pages_past_4gib():
    d = workloads.make_decode(6, 8, 2, 128, len_min=1, len_max=2500, seed=72, tail_fill="nan")
    say(f"[case] paged decode, pages past 4 GiB: lens={d['seq_lens'].tolist()}")
    kp, shift = far_pool(d["k_pages"])
    vp, _ = far_pool(d["v_pages"])
    o, lse = attn_paged_decode(dev(d["q"], "bf16"), kp, vp, shifted(d["block_table"], shift),
                               torch.from_numpy(d["seq_lens"]).cuda(), max_seq_len=d["max_seq_len"], scale=d["scale"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_decode(d["q"], d["k_pages"], d["v_pages"], d["block_table"], d["seq_lens"],
                                       d["scale"], dtype="bf16")
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, BF16_TOL, "paged decode past 4 GiB")
    del kp, vp
    torch.cuda.empty_cache()
