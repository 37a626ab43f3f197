"""Score modifications on the GPU against the fp64 oracle: a tanh soft cap
and ALiBi-style per-head slopes, alone and together, over every mask kind,
with sinks, in the bf16 prefill (d 128 and 64), the chunked prefill, the
paged decode and the fp32 prefill (the backward's are in the backward tests)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_io_aware_fwd_amd import attn_fwd, attn_paged_decode, attn_paged_prefill
from _gpu_helpers import BF16_SHARP_TOL, F32_TOL, compare, dev, doc_tensor, host_f64, say

pytestmark = pytest.mark.gpu


def alibi_slopes(Hq):
    """The geometric per-head slopes of ALiBi: 2^(-8 (h + 1) / Hq)."""
    return np.array([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=np.float32)


def prefill_case(c, label, softcap=0.0, slopes=None, sink_tokens=0, sinks=None, rows=None):
    say(f"[case] {label} B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} Nq={c['Nq']} Nk={c['Nk']} d={c['d']} "
        f"mask={c['mask']} window={c['window']} softcap={softcap} alibi={'yes' if slopes is not None else 'no'} "
        f"sink_tokens={sink_tokens} sinks={'yes' if sinks is not None else 'no'}")
    t = lambda a: None if a is None else torch.from_numpy(a).cuda()
    o, lse = attn_fwd(dev(c["q"], "bf16"), dev(c["k"], "bf16"), dev(c["v"], "bf16"), scale=c["scale"],
                      mask=c["mask"], window=c["window"], doc_offsets=doc_tensor(c), sink_tokens=sink_tokens,
                      sink_logits=t(sinks), softcap=softcap, alibi_slopes=t(slopes))
    torch.cuda.synchronize()
    f64 = lambda a: None if a is None else a.astype(np.float64)
    o_ref, l_ref = oracle.attention(oracle.to_f64(c["q"], "bf16"), oracle.to_f64(c["k"], "bf16"),
                                    oracle.to_f64(c["v"], "bf16"), c["scale"], c["mask"], c["window"],
                                    c["doc_offsets"], rows=rows, sink_tokens=sink_tokens, sink_logits=f64(sinks),
                                    softcap=softcap, alibi_slopes=f64(slopes))
    og, lg = host_f64(o), host_f64(lse)
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    return compare(og, lg, o_ref, l_ref, BF16_SHARP_TOL, label)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("mask,window,Nq,Nk", [("causal", 0, 700, 700), ("causal", 0, 300, 650),
                                               ("none", 0, 190, 333), ("window", 96, 600, 600),
                                               ("document", 0, 520, 520)])
@pytest.mark.parametrize("softcap,alibi", [(5.0, False), (0.0, True), (3.0, True)])
def test_prefill_score_mods(d, mask, window, Nq, Nk, softcap, alibi):
    # scale 4/sqrt(d): scores of a few units, so a cap of 3-5 bends most of them
    c = workloads.make_prefill(2, 8, 2, Nq, Nk, d, seed=91, mask=mask, window=window, doc_min=60, doc_max=200,
                               scale=4.0 / math.sqrt(d))
    prefill_case(c, f"mods {mask} {Nq}x{Nk} d{d}", softcap, alibi_slopes(8) if alibi else None)


def test_prefill_mods_with_sinks():
    c = workloads.make_prefill(1, 8, 2, 900, 900, 128, seed=93, mask="window", window=128, scale=0.3)
    sinks = np.random.default_rng(94).normal(0.0, 2.0, 8).astype(np.float32)
    prefill_case(c, "mods + window sinks", 4.0, alibi_slopes(8), sink_tokens=4, sinks=sinks)


def test_prefill_mods_bounds_every_score():
    # a cap of 0.25 on scores of tens of units: weights stay within e^{±0.5}
    # of each other, so each output row is close to the mean of its visible V rows
    c = workloads.make_prefill(1, 4, 4, 256, 256, 128, seed=95, mask="causal", scale=2.0)
    prefill_case(c, "cap 0.25, large scores", 0.25)


def test_prefill_negative_and_zero_slopes():
    c = workloads.make_prefill(1, 4, 2, 400, 400, 128, seed=96, mask="none")
    prefill_case(c, "mixed-sign slopes", 0.0, np.array([0.0, -0.05, 0.5, 1e-4], dtype=np.float32))


def test_prefill_mods_full_size_sampled_rows():
    """The 2048-token causal MHA workload (B 4, H 16, d 128) with a soft cap
    of 30 and ALiBi slopes, checked on seeded sampled rows of every head."""
    c = workloads.prefill_config("c2_causal_b4h16n2048")
    rows = np.unique(np.concatenate([np.arange(6), np.random.default_rng(97).integers(0, 2048, 40), [2047]]))
    prefill_case(c, "c2 + softcap 30 + alibi (sampled rows)", 30.0, alibi_slopes(16), rows=rows)


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("mask,window", [("causal", 0), ("window", 100)])
def test_chunked_prefill_score_mods(d, mask, window):
    c = workloads.make_chunked_prefill(6, 8, 2, d, chunks=[1, 40, 130, 300, 7, 64],
                                       prefixes=[0, 20, 500, 1000, 3, 2000], seed=98, tail_fill="nan")
    slopes = alibi_slopes(8)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    say(f"[case] chunked prefill mods d={d} {mask} {window}")
    o, lse = attn_paged_prefill(dev(c["q"], "bf16"), dev(c["k_pages"], "bf16"), dev(c["v_pages"], "bf16"),
                                i32(c["block_table"]), i32(c["seq_lens"]), i32(c["q_offsets"]),
                                max_seq_len=c["max_seq_len"], max_q_len=c["max_q_len"], scale=c["scale"], mask=mask,
                                window=window, softcap=2.5, alibi_slopes=torch.from_numpy(slopes).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_prefill(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                        c["q_offsets"], c["scale"], mask, window, dtype="bf16", softcap=2.5,
                                        alibi_slopes=slopes.astype(np.float64))
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, BF16_SHARP_TOL, f"chunked mods d{d} {mask}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask,window,Nq,Nk", [("causal", 0, 256, 256), ("none", 0, 100, 170),
                                               ("window", 40, 200, 230), ("document", 0, 256, 256)])
def test_fp32_prefill_score_mods(d, mask, window, Nq, Nk):
    # the fp32 path against the fp32 bound (max-abs 1e-5), soft cap and slopes together
    c = workloads.make_prefill(1, 4, 2, Nq, Nk, d, dtype="f32", seed=99, mask=mask, window=window, doc_min=30,
                               doc_max=120, scale=3.0 / math.sqrt(d))
    slopes = alibi_slopes(4)
    say(f"[case] fp32 mods {mask} {Nq}x{Nk} d{d}")
    o, lse = attn_fwd(dev(c["q"], "f32"), dev(c["k"], "f32"), dev(c["v"], "f32"), scale=c["scale"], mask=mask,
                      window=window, doc_offsets=doc_tensor(c), softcap=4.0,
                      alibi_slopes=torch.from_numpy(slopes).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(oracle.to_f64(c["q"], "f32"), oracle.to_f64(c["k"], "f32"),
                                    oracle.to_f64(c["v"], "f32"), c["scale"], mask, window, c["doc_offsets"],
                                    softcap=4.0, alibi_slopes=slopes.astype(np.float64))
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, F32_TOL, f"fp32 mods {mask} d{d}")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("softcap,alibi", [(2.0, False), (0.0, True), (1.5, True)])
def test_paged_decode_score_mods(d, softcap, alibi):
    # lengths around the 1024-key splits and the 16-token pages, an empty
    # sequence, GQA with a group of 4, NaN in every page tail
    c = workloads.make_decode(8, 8, 2, d, seq_lens=[0, 1, 15, 1023, 1025, 2048, 3001, 77], max_seq_len=3001,
                              seed=101, tail_fill="nan", scale=3.0 / math.sqrt(d))
    slopes = alibi_slopes(8) if alibi else None
    say(f"[case] decode mods d={d} softcap={softcap} alibi={alibi}")
    o, lse = attn_paged_decode(dev(c["q"], "bf16"), dev(c["k_pages"], "bf16"), dev(c["v_pages"], "bf16"),
                               torch.from_numpy(c["block_table"]).cuda(), torch.from_numpy(c["seq_lens"]).cuda(),
                               max_seq_len=c["max_seq_len"], scale=c["scale"], softcap=softcap,
                               alibi_slopes=None if slopes is None else torch.from_numpy(slopes).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_decode(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                       c["scale"], dtype="bf16", softcap=softcap,
                                       alibi_slopes=None if slopes is None else slopes.astype(np.float64))
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, BF16_SHARP_TOL, f"decode mods d{d}")


def test_paged_decode_mods_with_sinks():
    c = workloads.make_decode(5, 8, 2, 128, seq_lens=[3, 700, 1024, 2500, 40], max_seq_len=2500, seed=103,
                              tail_fill="nan")
    slopes, sinks = alibi_slopes(8), np.random.default_rng(104).normal(0.0, 2.0, 8).astype(np.float32)
    say("[case] decode mods + sinks")
    o, lse = attn_paged_decode(dev(c["q"], "bf16"), dev(c["k_pages"], "bf16"), dev(c["v_pages"], "bf16"),
                               torch.from_numpy(c["block_table"]).cuda(), torch.from_numpy(c["seq_lens"]).cuda(),
                               max_seq_len=c["max_seq_len"], scale=c["scale"], softcap=3.0,
                               alibi_slopes=torch.from_numpy(slopes).cuda(), sink_logits=torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_decode(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                       c["scale"], dtype="bf16", softcap=3.0, alibi_slopes=slopes.astype(np.float64),
                                       sink_logits=sinks.astype(np.float64))
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, BF16_SHARP_TOL, "decode mods + sinks")
