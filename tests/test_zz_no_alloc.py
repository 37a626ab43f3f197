"""The allocation-free paged decode (the library's own device scratch array)
against the workspace entry point: same kernels, so the outputs must agree
bit for bit, on two calls in a row with the second one smaller, and with
the scratch array left holding the first call's partials."""
import numpy as np
import pytest
import torch

import workloads
from exact_io_aware_fwd_amd import AttnError, attn_paged_decode, attn_paged_decode_noalloc
from _gpu_helpers import dev, say

pytestmark = pytest.mark.gpu


def to_dev(c):
    return dict(q=dev(c["q"], "bf16"), k=dev(c["k_pages"], "bf16"), v=dev(c["v_pages"], "bf16"),
                bt=torch.from_numpy(c["block_table"]).cuda(), sl=torch.from_numpy(c["seq_lens"]).cuda())


def both(c, **kw):
    t = to_dev(c)
    args = (t["q"], t["k"], t["v"], t["bt"], t["sl"])
    o_ref, l_ref = attn_paged_decode(*args, max_seq_len=c["max_seq_len"], scale=c["scale"], **kw)
    o = torch.full_like(t["q"], float("nan"))
    lse = torch.full((c["num_seqs"], c["Hq"]), float("nan"), dtype=torch.float32, device="cuda")
    attn_paged_decode_noalloc(*args, max_seq_len=c["max_seq_len"], scale=c["scale"], out=o, lse=lse, **kw)
    torch.cuda.synchronize()
    return o, lse, o_ref, l_ref


def test_noalloc_decode_matches_workspace_decode_on_two_calls():
    big = workloads.make_decode(24, 32, 8, 128, len_min=1, len_max=9000, seed=61, tail_fill="nan")
    small = workloads.make_decode(5, 8, 2, 128, seq_lens=[0, 1, 17, 1024, 1500], seed=62, tail_fill="nan")
    for label, c in (("first call, 24 sequences", big), ("second call, 5 smaller sequences", small)):
        say(f"[case] noalloc {label}: S={c['num_seqs']} Hq={c['Hq']} Hkv={c['Hkv']} max_len={c['max_seq_len']}")
        o, lse, o_ref, l_ref = both(c)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"{label}: O differs"
        assert torch.equal(lse, l_ref), f"{label}: LSE differs"


def test_noalloc_decode_with_sinks_and_mods_and_d64():
    c = workloads.make_decode(7, 8, 2, 64, len_min=1, len_max=3000, seed=63, tail_fill="nan")
    sinks = torch.from_numpy(np.random.default_rng(64).normal(0, 2, 8).astype(np.float32)).cuda()
    slopes = torch.from_numpy((2.0 ** (-np.arange(1, 9, dtype=np.float32)))).cuda()
    say(f"[case] noalloc d64 sinks+mods S={c['num_seqs']}")
    o, lse, o_ref, l_ref = both(c, sink_logits=sinks, softcap=4.0, alibi_slopes=slopes)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, l_ref)


def test_noalloc_decode_rejects_sizes_beyond_the_scratch_array():
    c = workloads.make_decode(2, 32, 8, 128, seq_lens=[10, 20], seed=65, with_values=False)
    q = dev(c["q"], "bf16")
    kp = torch.zeros((2, 8, 16, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((2, 8192), dtype=torch.int32, device="cuda")
    sl = torch.from_numpy(c["seq_lens"]).cuda()
    # 2 sequences x 32 heads x 128 splits of 1024 keys fit; 64 x 32 x 64 do not
    with pytest.raises(AttnError) as e:
        q64 = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
        attn_paged_decode_noalloc(q64, kp, kp, torch.zeros((64, 4096), dtype=torch.int32, device="cuda"),
                                  torch.zeros(64, dtype=torch.int32, device="cuda"), max_seq_len=65536)
    assert e.value.status == 3
    o, _ = attn_paged_decode_noalloc(q, kp, kp, bt, sl, max_seq_len=131072)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
