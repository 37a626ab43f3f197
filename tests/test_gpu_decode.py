"""Paged split-K decode parity on the GPU against the fp64 oracle, plus the
invariances the method must keep (page placement, workspace contents, runs)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_io_aware_fwd_amd import attn_paged_decode, attn_paged_decode_workspace_size
from _gpu_helpers import BF16_TOL, compare, dev, host_f64, parallel_map, say

pytestmark = pytest.mark.gpu


def to_dev(c):
    return dict(q=dev(c["q"], "bf16"), k=dev(c["k_pages"], "bf16"), v=dev(c["v_pages"], "bf16"),
                bt=torch.from_numpy(c["block_table"]).cuda(), sl=torch.from_numpy(c["seq_lens"]).cuda())


def run(c, t=None, workspace=None):
    t = t or to_dev(c)
    o, lse = attn_paged_decode(t["q"], t["k"], t["v"], t["bt"], t["sl"], max_seq_len=c["max_seq_len"],
                               scale=c["scale"], workspace=workspace)
    torch.cuda.synchronize()
    return o, lse


def check(c, label, seqs=None):
    say(f"[case] {label} S={c['num_seqs']} Hq={c['Hq']} Hkv={c['Hkv']} d={c['d']} lens={c['seq_lens'][:8].tolist()}")
    o, lse = run(c)
    og, lg = host_f64(o), host_f64(lse)
    o_ref, l_ref = oracle.paged_decode(c["q"], c["k_pages"], c["v_pages"], c["block_table"], c["seq_lens"],
                                       c["scale"], seqs=seqs, dtype="bf16")
    if seqs is not None:
        og, lg = og[list(seqs)], lg[list(seqs)]
    return compare(og, lg, o_ref, l_ref, BF16_TOL, label)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 1), (32, 2), (6, 2), (2, 2)])
def test_decode_small(d, Hq, Hkv):
    lens = [0, 1, 15, 16, 17, 511, 512, 513, 1500, 1024]
    c = workloads.make_decode(len(lens), Hq, Hkv, d, seq_lens=lens, max_seq_len=1600, seed=21,
                              tail_fill="nan", extra_pages=5)
    check(c, f"decode d{d} Hq{Hq} Hkv{Hkv}")


def test_decode_random_lengths_nan_tails():
    c = workloads.make_decode(24, 32, 8, 128, len_min=1, len_max=5000, seed=23, tail_fill="nan")
    check(c, "decode random lens")


def test_decode_page_permutation_invariance():
    c = workloads.make_decode(6, 8, 2, 128, len_min=100, len_max=3000, seed=25, extra_pages=4)
    o1, l1 = run(c)
    pi = np.random.default_rng(26).permutation(c["k_pages"].shape[0])
    c2 = dict(c)
    for key in ("k_pages", "v_pages"):
        arr = np.empty_like(c[key])
        arr[pi] = c[key]
        c2[key] = arr
    bt = c["block_table"].copy()
    valid = bt >= 0
    bt[valid] = pi[bt[valid]]
    c2["block_table"] = bt
    o2, l2 = run(c2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_workspace_contents_and_determinism():
    c = workloads.make_decode(5, 8, 2, 128, len_min=10, len_max=2000, seed=27)
    t = to_dev(c)
    need = attn_paged_decode_workspace_size(5, 8, 128, c["max_seq_len"])
    ws = torch.full((need // 4 + 1,), float("nan"), dtype=torch.float32, device="cuda")
    o1, l1 = run(c, t, workspace=ws.view(torch.uint8)[:need])
    o2, l2 = run(c, t)
    o3, l3 = run(c, t)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o2, o3) and torch.equal(l2, l3)


@pytest.mark.slow
def test_config_paged_decode_64_all_sequences():
    """All 64 sequences of the decode workload, in the launch configuration
    the benchmark times; the oracle takes one sequence per host thread."""
    c = workloads.decode_config("c5_paged_decode_64")
    say(f"[case] c5 S={c['num_seqs']} Hq={c['Hq']} Hkv={c['Hkv']} d={c['d']} tokens={int(c['seq_lens'].sum())}")
    o, lse = run(c)
    og, lg = host_f64(o), host_f64(lse)
    parts = parallel_map(lambda s: oracle.paged_decode(c["q"], c["k_pages"], c["v_pages"], c["block_table"],
                                                       c["seq_lens"], c["scale"], seqs=[s], dtype="bf16"),
                         range(c["num_seqs"]), "c5")
    o_ref = np.concatenate([p[0] for p in parts])
    l_ref = np.concatenate([p[1] for p in parts])
    compare(og, lg, o_ref, l_ref, BF16_TOL, "c5 all 64 sequences")


def test_decode_lengths_past_max_seq_len_are_clamped():
    """seq_lens entries above max_seq_len break the caller contract; the
    kernels clamp them, so the result is that of the clamped lengths and
    neither pass reads or writes outside the workspace (NaN guard bands)."""
    lens = [100, 3000, 2050]
    c = workloads.make_decode(len(lens), 8, 2, 128, seq_lens=lens, max_seq_len=3000, seed=29)
    t = to_dev(c)
    max_len = 2048
    need = attn_paged_decode_workspace_size(len(lens), 8, 128, max_len)
    guard = 4096
    buf = torch.full(((need + 2 * guard) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    ws = buf.view(torch.uint8)[guard:guard + need]
    o, lse = attn_paged_decode(t["q"], t["k"], t["v"], t["bt"], t["sl"], max_seq_len=max_len, scale=c["scale"],
                               workspace=ws)
    torch.cuda.synchronize()
    raw = buf.view(torch.uint8)
    assert torch.isnan(raw[:guard].view(torch.float32)).all(), "write before the workspace"
    assert torch.isnan(raw[guard + need:].view(torch.float32)).all(), "write past the workspace"
    clamped = np.minimum(c["seq_lens"], max_len)
    o_ref, l_ref = oracle.paged_decode(c["q"], c["k_pages"], c["v_pages"], c["block_table"], clamped, c["scale"],
                                       dtype="bf16")
    compare(host_f64(o), host_f64(lse), o_ref, l_ref, BF16_TOL, "decode lengths clamped to max_seq_len")


def test_caller_buffers_are_checked():
    """Wrong out= / lse= / workspace arguments raise before any launch."""
    c = workloads.make_decode(2, 8, 2, 128, seq_lens=[40, 70], seed=30)
    t = to_dev(c)
    kw = dict(max_seq_len=c["max_seq_len"], scale=c["scale"])
    bad_out = [torch.empty((2, 8, 64), dtype=torch.bfloat16, device="cuda"),
               torch.empty((2, 8, 128), dtype=torch.float32, device="cuda"),
               torch.empty((2, 8, 256), dtype=torch.bfloat16, device="cuda")[:, :, ::2],
               torch.empty((2, 8, 128), dtype=torch.bfloat16)]
    for out in bad_out:
        with pytest.raises(ValueError):
            attn_paged_decode(t["q"], t["k"], t["v"], t["bt"], t["sl"], out=out, **kw)
    for lse in [torch.empty((2, 7), dtype=torch.float32, device="cuda"),
                torch.empty((2, 8), dtype=torch.bfloat16, device="cuda")]:
        with pytest.raises(ValueError):
            attn_paged_decode(t["q"], t["k"], t["v"], t["bt"], t["sl"], lse=lse, **kw)
    with pytest.raises(ValueError):
        attn_paged_decode(t["q"], t["k"], t["v"], t["bt"], t["sl"], workspace=torch.empty(1 << 20, dtype=torch.uint8),
                          **kw)
    # a too-small workspace is the library's own error
    with pytest.raises(RuntimeError):
        attn_paged_decode(t["q"], t["k"], t["v"], t["bt"], t["sl"],
                          workspace=torch.empty(16, dtype=torch.uint8, device="cuda"), **kw)
