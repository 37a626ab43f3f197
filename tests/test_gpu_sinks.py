"""Attention sinks on the GPU against the fp64 oracle: sink tokens beside a
sliding window, and a learned sink logit per query head, in the prefill
(bf16 and fp32), chunked-prefill and decode paths."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_io_aware_fwd_amd import attn_fwd, attn_paged_decode, attn_paged_prefill
from _gpu_helpers import BF16_TOL, F32_TOL, compare, dev, doc_tensor, host_f64, oracle_prefill, say

pytestmark = pytest.mark.gpu


def sink_values(Hq, seed):
    """Per-head sink logits: ordinary values plus one that dominates every
    score and one far below them."""
    s = np.random.default_rng(seed).normal(0.0, 2.0, Hq)
    s[0], s[-1] = 30.0, -30.0
    return s.astype(np.float32)


def prefill_case(case, label, sink_tokens=0, sinks=None, rows=None):
    dt = case["dtype"]
    say(f"[case] {label} B={case['B']} Hq={case['Hq']} Hkv={case['Hkv']} Nq={case['Nq']} Nk={case['Nk']} "
        f"d={case['d']} mask={case['mask']} window={case['window']} sink_tokens={sink_tokens} "
        f"sinks={'yes' if sinks is not None else 'no'}")
    sl = None if sinks is None else torch.from_numpy(sinks).cuda()
    o, lse = attn_fwd(dev(case["q"], dt), dev(case["k"], dt), dev(case["v"], dt), scale=case["scale"],
                      mask=case["mask"], window=case["window"], doc_offsets=doc_tensor(case),
                      sink_tokens=sink_tokens, sink_logits=sl)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(oracle.to_f64(case["q"], dt), oracle.to_f64(case["k"], dt),
                                    oracle.to_f64(case["v"], dt), case["scale"], case["mask"], case["window"],
                                    case["doc_offsets"], rows=rows, sink_tokens=sink_tokens,
                                    sink_logits=None if sinks is None else sinks.astype(np.float64))
    og, lg = host_f64(o), host_f64(lse)
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    return compare(og, lg, o_ref, l_ref, F32_TOL if dt == "f32" else BF16_TOL, label)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("sink_tokens", [1, 4, 64, 100, 300])
@pytest.mark.parametrize("with_logits", [False, True])
def test_window_with_sink_tokens(d, sink_tokens, with_logits):
    c = workloads.make_prefill(1, 8, 2, 1000, 1000, d, seed=51, mask="window", window=128)
    prefill_case(c, f"window128 sinks{sink_tokens} d{d}", sink_tokens,
                 sink_values(8, 52) if with_logits else None)


@pytest.mark.parametrize("mask,window,Nq,Nk", [("causal", 0, 700, 700), ("causal", 0, 300, 200),
                                               ("none", 0, 130, 520), ("window", 64, 600, 600),
                                               ("document", 0, 800, 800)])
def test_learned_sink_logits(mask, window, Nq, Nk):
    c = workloads.make_prefill(2, 8, 4, Nq, Nk, 128, seed=53, mask=mask, window=window, doc_min=100, doc_max=300)
    prefill_case(c, f"sink logits {mask} {Nq}x{Nk}", 0, sink_values(8, 54))


def test_sink_logits_fp32():
    c = workloads.make_prefill(1, 4, 2, 256, 256, 64, dtype="f32", seed=55, mask="window", window=40)
    prefill_case(c, "fp32 window40 sinks", 7, sink_values(4, 56))


def test_minus_inf_sink_is_no_sink():
    c = workloads.make_prefill(1, 8, 2, 500, 500, 128, seed=57, mask="causal")
    q, k, v = dev(c["q"], "bf16"), dev(c["k"], "bf16"), dev(c["v"], "bf16")
    o1, l1 = attn_fwd(q, k, v, scale=c["scale"], mask="causal")
    o2, l2 = attn_fwd(q, k, v, scale=c["scale"], mask="causal",
                      sink_logits=torch.full((8,), -float("inf"), device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_decode_sink_logits():
    c = workloads.make_decode(9, 8, 2, 128, seq_lens=[0, 1, 17, 511, 513, 1500, 40, 3000, 2],
                              max_seq_len=3000, seed=59, tail_fill="nan")
    sinks = sink_values(8, 60)
    say("[case] decode with sink logits")
    o, lse = attn_paged_decode(dev(c["q"], "bf16"), dev(c["k_pages"], "bf16"), dev(c["v_pages"], "bf16"),
                               torch.from_numpy(c["block_table"]).cuda(), torch.from_numpy(c["seq_lens"]).cuda(),
                               max_seq_len=c["max_seq_len"], scale=c["scale"],
                               sink_logits=torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_decode(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                       c["scale"], dtype="bf16", sink_logits=sinks.astype(np.float64))
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, BF16_TOL, "decode sinks")


@pytest.mark.parametrize("mask,window,sink_tokens", [("window", 100, 5), ("window", 64, 200), ("causal", 0, 0)])
def test_chunked_prefill_sinks(mask, window, sink_tokens):
    c = workloads.make_chunked_prefill(6, 8, 2, 128, chunks=[1, 40, 130, 300, 7, 64],
                                       prefixes=[0, 20, 500, 1000, 3, 2000], seed=61, tail_fill="nan")
    sinks = sink_values(8, 62)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    say(f"[case] chunked prefill sinks {mask} {window} {sink_tokens}")
    o, lse = attn_paged_prefill(dev(c["q"], "bf16"), dev(c["k_pages"], "bf16"), dev(c["v_pages"], "bf16"),
                                i32(c["block_table"]), i32(c["seq_lens"]), i32(c["q_offsets"]),
                                max_seq_len=c["max_seq_len"], max_q_len=c["max_q_len"], scale=c["scale"], mask=mask,
                                window=window, sink_tokens=sink_tokens, sink_logits=torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_prefill(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                        c["q_offsets"], c["scale"], mask, window, dtype="bf16",
                                        sink_tokens=sink_tokens, sink_logits=sinks.astype(np.float64))
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, BF16_TOL, f"chunked sinks {mask}")


def test_window_sinks_full_size_sampled_rows():
    """The 8192-token GQA window-1024 workload with 4 sink tokens and learned
    sinks, checked on a seeded sample of rows (the first rows, the rows where
    the window leaves the sinks behind, and random rows)."""
    c = workloads.prefill_config("c3b_gqa_window1024_n8192")
    rows = np.unique(np.concatenate([np.arange(8), np.arange(1020, 1036),
                                     np.random.default_rng(63).integers(0, 8192, 48), [8191]]))
    prefill_case(c, "c3b + sinks (sampled rows)", 4, sink_values(32, 64), rows=rows)
