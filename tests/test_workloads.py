"""The seeded generators: determinism, bf16 rounding and layout."""
import numpy as np
import pytest
import torch

import workloads


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -1e-40, np.inf, -np.inf],
                                 dtype=np.float32)])
    ours = workloads.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nan = workloads.bf16_bits_from_f32(np.array([np.nan], dtype=np.float32))
    assert (int(nan[0]) & 0x7F80) == 0x7F80 and (int(nan[0]) & 0x7F) != 0


def test_prefill_generator_is_deterministic_and_shaped():
    a = workloads.make_prefill(2, 4, 2, 33, 40, 64, seed=5, mask="causal")
    b = workloads.make_prefill(2, 4, 2, 33, 40, 64, seed=5, mask="causal")
    for key in ("q", "k", "v"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (2, 4, 33, 64) and a["k"].shape == (2, 2, 40, 64)
    assert a["q"].dtype == np.uint16
    c = workloads.make_prefill(2, 4, 2, 33, 40, 64, seed=6, mask="causal")
    assert not np.array_equal(a["q"], c["q"])
    assert a["scale"] == pytest.approx(1 / 8)


def test_document_lengths_fill_the_sequence():
    c = workloads.make_prefill(1, 2, 1, 32768, 32768, 8, seed=0, mask="document", doc_min=512, doc_max=8192)
    off = c["doc_offsets"]
    assert off[0] == 0 and off[-1] == 32768 and np.all(np.diff(off) > 0)
    lens = np.diff(off)
    assert np.all(lens[:-1] >= 512) and np.all(lens <= 8192)
    assert lens.tolist() == [7045, 5404, 4438, 2584, 2876, 826, 1089, 638, 1858, 6010]


def test_decode_generator_layout():
    c = workloads.make_decode(5, 8, 2, 16, len_min=1, len_max=50, seed=2, extra_pages=3)
    bt, lens = c["block_table"], c["seq_lens"]
    used = [bt[s, : -(-int(n) // 16)] for s, n in enumerate(lens)]
    allp = np.concatenate(used)
    assert len(set(allp.tolist())) == allp.size          # no page shared
    assert c["k_pages"].shape[0] == allp.size + 3
    for s, n in enumerate(lens):
        assert np.all(bt[s, -(-int(n) // 16):] == -1)
        last = bt[s, (int(n) - 1) // 16]
        tail = int(n) % 16
        if tail:
            assert np.all(c["k_pages"][last, :, tail:] == 0)


def test_chunked_prefill_structure():
    c = workloads.make_chunked_prefill(6, 4, 2, 16, prefix_min=0, prefix_max=100, chunk_min=1, chunk_max=40,
                                       seed=2, tail_fill="nan")
    offs, lens, bt = c["q_offsets"], c["seq_lens"], c["block_table"]
    chunks = np.diff(offs)
    assert offs[0] == 0 and np.all(chunks >= 1) and c["q"].shape == (offs[-1], 4, 16)
    assert np.all(lens >= chunks) and c["max_q_len"] == chunks.max()
    P = c["page_size"]
    used = np.concatenate([bt[s, :-(-int(n) // P)] for s, n in enumerate(lens)])
    assert used.size == c["k_pages"].shape[0] and np.unique(used).size == used.size   # each page once
    for s, n in enumerate(lens):
        assert np.all(bt[s, -(-int(n) // P):] == -1)
        if n % P:   # slots past the end hold the NaN fill
            tail = c["k_pages"][bt[s, n // P], :, n % P:, :]
            assert np.all(tail == workloads.gen.BF16_QNAN)


def test_chunked_config_c6_shape():
    c = workloads.chunked_config("c6_chunked_prefill_16")
    assert c["q_offsets"][-1] == c["q"].shape[0] and c["num_seqs"] == 16
    assert c["k_pages"].shape[1:] == (8, 16, 128)
    assert int(c["max_seq_len"]) == int(c["seq_lens"].max())
