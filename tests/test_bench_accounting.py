"""Host-side work accounting of the benchmark, checked against the oracle's
mask and against the decode byte arithmetic on the attention pages."""
import numpy as np
import pytest

import bench
import oracle
import workloads


@pytest.mark.parametrize("Nq,Nk,mask,window,offs", [
    (37, 37, "none", 0, None), (37, 37, "causal", 0, None), (20, 50, "causal", 0, None), (50, 20, "causal", 0, None),
    (64, 64, "window", 5, None), (30, 60, "window", 17, None), (40, 40, "document", 0, [0, 3, 4, 20, 40]),
])
def test_visible_pairs_matches_oracle_mask(Nq, Nk, mask, window, offs):
    assert bench.visible_pairs(Nq, Nk, mask, window, offs) == int(oracle.visibility(Nq, Nk, mask, window, offs).sum())


def test_config_pair_counts():
    assert bench.visible_pairs(2048, 2048, "causal") == 2_098_176
    assert bench.visible_pairs(8192, 8192, "causal") == 33_558_528
    assert bench.visible_pairs(8192, 8192, "window", 1024) == 7_864_832
    c = workloads.make_prefill(1, 1, 1, 32768, 32768, 8, mask="document", doc_min=512, doc_max=8192, seed=0)
    assert bench.visible_pairs(32768, 32768, "document", 0, c["doc_offsets"]) == 77_679_895


def test_decode_bytes_match_the_pages_arithmetic():
    # "Attention Is the Bottleneck", Prefill and decode: a Llama-3-8B-shaped KV
    # cache (8 KV heads, head dim 128, bf16) holds 2*8*128*2 = 4096 bytes per
    # token per layer; x 32 layers = 131,072 bytes = 128 KiB per token.
    c = dict(seq_lens=np.array([32768]), num_seqs=1, Hq=32, Hkv=8, d=128, page_size=16)
    kv = bench.decode_bytes(c) - (2 * 32 * 128 * 2 + 32 * 4 + 2048 * 4 + 4)
    assert kv == 32768 * 4096
    assert kv * 32 == 4 * 2**30              # 4 GiB per generated token at 32K context, all 32 layers
    assert kv * 32 / 3.35e12 == pytest.approx(1.28e-3, rel=0.01)   # ~1.3 ms at 3.35 TB/s


def test_decode_config_bytes():
    c = workloads.decode_config("c5_paged_decode_64", with_values=False)
    assert int(c["seq_lens"].sum()) == 1_101_299
    assert bench.decode_bytes(c) == 4_512_253_168


def test_chunked_visible_pairs_closed_form():
    # causal chunk of n queries at the end of L cached keys: query i sees
    # L - n + i + 1 keys, so the chunk sees n (L - n) + n (n + 1) / 2 pairs
    c = workloads.chunked_config("c6_chunked_prefill_16")
    n = np.diff(c["q_offsets"]).astype(np.int64)
    L = c["seq_lens"].astype(np.int64)
    assert bench.chunked_visible_pairs(c) == int(np.sum(n * (L - n) + n * (n + 1) // 2))
    assert bench.chunked_flops(c) == 4 * 128 * 32 * bench.chunked_visible_pairs(c)


def test_pmc_plan_maps_dispatches_to_workloads():
    """A dispatch's workload follows from its kernel and its rank among that
    kernel's dispatches in the counter pass; other kernels are ignored and a
    count that does not match the plan is an error."""
    per = {}
    did = 0
    names = {"prefill_bf16_kernel<128, false>": "void xattn::prefill_bf16_kernel<128, false>(xattn::PrefillParams)",
             "prefill_bf16_k32_kernel<false>": "void xattn::prefill_bf16_k32_kernel<false>(xattn::PrefillParams)",
             "decode_split_kernel<128, false>": "void xattn::decode_split_kernel<128, false>(xattn::DecodeParams)",
             "decode_combine_kernel<128>": "void xattn::decode_combine_kernel<128>(xattn::DecodeParams)",
             "paged_prefill_swz_kernel<false>": "void xattn::paged_prefill_swz_kernel<false>(xattn::PagedPrefillParams)",
             "bwd_dq_kernel": "void xattn::bwd_dq_kernel(xattn::BwdParams)",
             "bwd_dkdv2_kernel": "void xattn::bwd_dkdv2_kernel(xattn::BwdParams)"}
    per[(str(did), "__amd_rocclr_copyBuffer")] = 1.0
    for leg, n in bench.PMC_PLAN:
        for i in range(n):
            for k in bench.LEG_KERNELS[leg]:
                did += 1
                per[(str(did), names[k])] = float(100 * did)
                did += 1
                per[(str(did), "void at::native::elementwise_kernel<...>(int)")] = -1.0
    got = bench._by_leg(per)
    assert set(got) == {leg for leg, _ in bench.PMC_PLAN}
    assert len(got["c3a"]["prefill_bf16_kernel<128, false>"]) == 2
    assert got["c2"]["prefill_bf16_kernel<128, false>"][0] == 100.0     # the first dispatch of the pass
    assert set(got["c4"]) == {"prefill_bf16_k32_kernel<false>"}         # window and document legs
    assert all(v > 0 for leg in got.values() for vals in leg.values() for v in vals)
    del per[max(per, key=lambda k: int(k[0]) if "bwd_dkdv" in k[1] else -1)]
    with pytest.raises(SystemExit):
        bench._by_leg(per)
