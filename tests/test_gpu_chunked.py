"""Chunked prefill over the paged cache: GPU parity against the fp64 oracle,
equality with the contiguous prefill kernel when a chunk is a whole
sequence, page-placement invariance, and sampled rows at the full workload."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_io_aware_fwd_amd import attn_fwd, attn_paged_prefill
from _gpu_helpers import BF16_TOL, compare, dev, host_f64, parallel_map, say

pytestmark = pytest.mark.gpu


def to_dev(c):
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    return dict(q=dev(c["q"], "bf16"), k=dev(c["k_pages"], "bf16"), v=dev(c["v_pages"], "bf16"),
                bt=i32(c["block_table"]), sl=i32(c["seq_lens"]), qo=i32(c["q_offsets"]))


def run(c, t=None, mask="causal", window=0):
    t = t or to_dev(c)
    o, lse = attn_paged_prefill(t["q"], t["k"], t["v"], t["bt"], t["sl"], t["qo"], max_seq_len=c["max_seq_len"],
                                max_q_len=c["max_q_len"], scale=c["scale"], mask=mask, window=window)
    torch.cuda.synchronize()
    return o, lse


def check(c, label, mask="causal", window=0):
    say(f"[case] {label} S={c['num_seqs']} Hq={c['Hq']} Hkv={c['Hkv']} d={c['d']} mask={mask} "
        f"lens={c['seq_lens'][:8].tolist()} chunks={np.diff(c['q_offsets'])[:8].tolist()}")
    o, lse = run(c, mask=mask, window=window)
    o_ref, l_ref = oracle.paged_prefill(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                        c["q_offsets"], c["scale"], mask, window, dtype="bf16")
    return compare(host_f64(o), host_f64(lse), o_ref, l_ref, BF16_TOL, label)


# chunk lengths cover one token, a page, a ragged 128-row query tile and
# several tiles; prefixes cover empty, sub-page, page-aligned and long contexts
CHUNKS = [1, 16, 130, 300, 64, 257, 5, 3]
PREFIXES = [0, 7, 16, 1000, 513, 0, 4000, 0]


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("mask,window", [("causal", 0), ("none", 0), ("window", 100)])
def test_chunked_small(d, mask, window):
    c = workloads.make_chunked_prefill(len(CHUNKS), 8, 2, d, chunks=CHUNKS, prefixes=PREFIXES, seed=31,
                                       tail_fill="nan", extra_pages=3)
    check(c, f"chunked d{d} {mask}", mask, window)


def test_chunked_empty_cache_rows_see_nothing():
    # seq 1 has no cached key at all, seq 2's chunk is longer than its cache
    c = workloads.make_chunked_prefill(3, 4, 1, 128, chunks=[40, 20, 50], prefixes=[10, 0, 0], seed=33,
                                       tail_fill="nan")
    c["seq_lens"] = np.array([50, 0, 30], dtype=np.int32)   # chunks of 20 and 50 rows over 0 and 30 keys
    check(c, "chunked empty / short cache")


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (4, 4), (6, 2)])
def test_chunked_random_gqa(Hq, Hkv):
    c = workloads.make_chunked_prefill(10, Hq, Hkv, 128, prefix_min=0, prefix_max=3000, chunk_min=1,
                                       chunk_max=700, seed=35, tail_fill="nan")
    check(c, f"chunked random Hq{Hq} Hkv{Hkv}")


def test_whole_sequence_chunk_equals_contiguous_prefill():
    # a chunk that is the whole sequence is plain causal prefill: the two
    # kernels share the tile computation and tile boundaries, so the outputs
    # agree bit for bit
    lens = [700, 1024, 129]
    c = workloads.make_chunked_prefill(len(lens), 8, 2, 128, chunks=lens, prefixes=[0] * len(lens), seed=37,
                                       tail_fill="nan")
    o, lse = run(c)
    for s, n in enumerate(lens):
        k = oracle.gather_sequence(c["k_pages"], c["block_table"][s], n)[None]     # [1, Hkv, n, d] bits
        v = oracle.gather_sequence(c["v_pages"], c["block_table"][s], n)[None]
        a, b = c["q_offsets"][s], c["q_offsets"][s + 1]
        q = np.ascontiguousarray(np.transpose(c["q"][a:b], (1, 0, 2)))[None]         # [1, Hq, n, d]
        od, ld = attn_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), scale=c["scale"], mask="causal")
        torch.cuda.synchronize()
        op = o[a:b].permute(1, 0, 2).unsqueeze(0)
        lp = lse[a:b].permute(1, 0).unsqueeze(0)
        assert torch.equal(op.view(torch.int16), od.view(torch.int16)), f"seq {s}: O differs"
        assert torch.equal(lp, ld), f"seq {s}: LSE differs"


def test_chunked_page_permutation_invariance():
    c = workloads.make_chunked_prefill(5, 8, 2, 128, prefix_min=0, prefix_max=2000, chunk_min=50, chunk_max=400,
                                       seed=39, extra_pages=6)
    o1, l1 = run(c)
    pi = np.random.default_rng(40).permutation(c["k_pages"].shape[0])
    c2 = dict(c)
    for key in ("k_pages", "v_pages"):
        arr = np.empty_like(c[key])
        arr[pi] = c[key]
        c2[key] = arr
    bt = c["block_table"].copy()
    bt[bt >= 0] = pi[bt[bt >= 0]]
    c2["block_table"] = bt
    o2, l2 = run(c2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.slow
def test_chunked_full_workload_all_rows():
    """The 16-sequence workload at full size, in the launch configuration the
    benchmark times; every row of every chunk and head is compared with the
    oracle, one (sequence, query head) per host thread: each sequence is an
    attention problem of its own with Nq = chunk, Nk = cached length, and
    query head h reads KV head h // (Hq / Hkv)."""
    c = workloads.chunked_config("c6_chunked_prefill_16")
    say(f"[case] c6 S={c['num_seqs']} Hq={c['Hq']} Hkv={c['Hkv']} chunk tokens={int(c['q_offsets'][-1])} "
        f"cached={int(c['seq_lens'].sum())}")
    o, lse = run(c)
    og, lg = host_f64(o), host_f64(lse)
    S, Hq, g = c["num_seqs"], c["Hq"], c["Hq"] // c["Hkv"]
    offs, lens = c["q_offsets"], c["seq_lens"]
    kv = parallel_map(lambda s: (oracle.from_bf16_bits(oracle.gather_sequence(c["k_pages"], c["block_table"][s],
                                                                              int(lens[s]))),
                                 oracle.from_bf16_bits(oracle.gather_sequence(c["v_pages"], c["block_table"][s],
                                                                              int(lens[s])))),
                      range(S), "c6 gather")
    o_ref = np.empty_like(og)
    l_ref = np.empty_like(lg)

    def one(task):
        s, h = task
        a, b = int(offs[s]), int(offs[s + 1])
        q = np.transpose(oracle.to_f64(c["q"][a:b, h:h + 1], "bf16"), (1, 0, 2))[None]     # [1, 1, n, d]
        k, v = kv[s][0][h // g:h // g + 1][None], kv[s][1][h // g:h // g + 1][None]
        ob, lb = oracle.attention(q, k, v, c["scale"], "causal")
        o_ref[a:b, h], l_ref[a:b, h] = ob[0, 0], lb[0, 0]

    work = lambda t: -(int(offs[t[0] + 1]) - int(offs[t[0]])) * int(lens[t[0]])
    parallel_map(one, sorted(((s, h) for s in range(S) for h in range(Hq)), key=work), "c6")
    compare(og, lg, o_ref, l_ref, BF16_TOL, f"c6 all {int(offs[-1])} rows of {Hq} heads")
