"""Prefill parity on the GPU: the HIP kernels against the fp64 oracle.

Tolerances: fp32 max-abs 1e-5 on O; bf16 max-abs 1e-2 and mean-abs 1e-3 on
O; LSE max-abs 1e-3; rows that see no key exactly O = 0, LSE = -inf.
"""
import numpy as np
import pytest
import torch

import workloads
from exact_io_aware_fwd_amd import attn_fwd
from _gpu_helpers import (BF16_TOL, F32_TOL, compare, dev, doc_tensor, host_f64, oracle_document_by_parts,
                          oracle_prefill, oracle_prefill_by_head, say)

pytestmark = pytest.mark.gpu


def run_case(case, rows=None, label=""):
    dt = case["dtype"]
    say(f"[case] {label} B={case['B']} Hq={case['Hq']} Hkv={case['Hkv']} Nq={case['Nq']} Nk={case['Nk']} "
        f"d={case['d']} {dt} mask={case['mask']} W={case['window']}")
    q, k, v = dev(case["q"], dt), dev(case["k"], dt), dev(case["v"], dt)
    o, lse = attn_fwd(q, k, v, scale=case["scale"], mask=case["mask"], window=case["window"],
                      doc_offsets=doc_tensor(case))
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_prefill(case, rows=rows)
    og, lg = host_f64(o), host_f64(lse)
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    return compare(og, lg, o_ref, lse_ref, F32_TOL if dt == "f32" else BF16_TOL, label)


def test_single_head_f32_config():
    case = workloads.prefill_config("c1_f32_single_head")
    run_case(case, label="c1")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 37)])
def test_f32_small(d, mask, window):
    case = workloads.make_prefill(2, 4, 2, 200, 200, d, dtype="f32", seed=11, mask=mask, window=window)
    run_case(case, label=f"f32 d{d} {mask}")


SHAPES = [1, 31, 64, 65, 128, 129, 300, 1000]


@pytest.mark.parametrize("N", SHAPES)
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_bf16_ragged_lengths(N, mask):
    case = workloads.make_prefill(2, 4, 2, N, N, 128, seed=N, mask=mask)
    run_case(case, label=f"bf16 N{N} {mask}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 1), ("window", 7),
                                         ("window", 200), ("window", 5000)])
def test_bf16_masks(d, mask, window):
    case = workloads.make_prefill(1, 8, 2, 777, 777, d, seed=3, mask=mask, window=window)
    run_case(case, label=f"bf16 d{d} {mask} W{window}")


@pytest.mark.parametrize("lens", [[100, 1, 50, 149], [300], [64, 64, 64, 64, 10], [1] * 20 + [280]])
def test_bf16_document(lens):
    N = sum(lens)
    case = workloads.make_prefill(2, 4, 1, N, N, 128, seed=5, mask="document", doc_lens=lens)
    run_case(case, label=f"bf16 doc {lens[:5]}")


@pytest.mark.parametrize("Nq,Nk,mask", [(100, 300, "causal"), (300, 100, "causal"), (1, 500, "causal"),
                                        (50, 400, "window"), (200, 77, "none"), (129, 1, "none")])
def test_bf16_unequal_lengths(Nq, Nk, mask):
    case = workloads.make_prefill(1, 4, 4, Nq, Nk, 128, seed=7, mask=mask, window=60)
    run_case(case, label=f"bf16 Nq{Nq} Nk{Nk} {mask}")


def test_bf16_mqa():
    case = workloads.make_prefill(1, 8, 1, 333, 333, 128, seed=9, mask="causal")
    run_case(case, label="bf16 mqa")


def test_outputs_written_in_place_only():
    """Guard bands around o and lse stay untouched, q/k/v stay unchanged."""
    case = workloads.make_prefill(1, 4, 2, 130, 130, 128, seed=13, mask="causal")
    q, k, v = dev(case["q"], "bf16"), dev(case["k"], "bf16"), dev(case["v"], "bf16")
    q0, k0, v0 = q.clone(), k.clone(), v.clone()
    n = q.numel()
    obuf = torch.full((n + 2048,), float("nan"), dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((4 * 130 + 128,), float("nan"), dtype=torch.float32, device="cuda")
    o = obuf[1024:1024 + n].view(q.shape)
    lse = lbuf[64:64 + 4 * 130].view(1, 4, 130)
    attn_fwd(q, k, v, mask="causal", out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(obuf[:1024]).all() and torch.isnan(obuf[1024 + n:]).all()
    assert torch.isnan(lbuf[:64]).all() and torch.isnan(lbuf[64 + 4 * 130:]).all()
    assert torch.equal(q, q0) and torch.equal(k, k0) and torch.equal(v, v0)
    assert torch.isfinite(o.float()).all()


def test_deterministic_run_to_run():
    case = workloads.make_prefill(2, 8, 2, 1000, 1000, 128, seed=17, mask="causal")
    q, k, v = dev(case["q"], "bf16"), dev(case["k"], "bf16"), dev(case["v"], "bf16")
    o1, l1 = attn_fwd(q, k, v, mask="causal")
    o2, l2 = attn_fwd(q, k, v, mask="causal")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_lse_optional():
    case = workloads.make_prefill(1, 2, 2, 100, 100, 64, seed=19, mask="causal")
    q, k, v = dev(case["q"], "bf16"), dev(case["k"], "bf16"), dev(case["v"], "bf16")
    o1, _ = attn_fwd(q, k, v, mask="causal", with_lse=False)
    o2, _ = attn_fwd(q, k, v, mask="causal")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_caller_buffers_are_checked():
    """Wrong out= / lse= arguments raise before any launch: the library sees
    only pointers and would write past a short buffer."""
    case = workloads.make_prefill(1, 4, 2, 130, 130, 128, seed=14, mask="causal")
    q, k, v = dev(case["q"], "bf16"), dev(case["k"], "bf16"), dev(case["v"], "bf16")
    bad_out = [torch.empty((1, 4, 129, 128), dtype=torch.bfloat16, device="cuda"),
               torch.empty((1, 4, 130, 128), dtype=torch.float32, device="cuda"),
               torch.empty((1, 4, 130, 256), dtype=torch.bfloat16, device="cuda")[..., ::2],
               torch.empty((1, 4, 130, 128), dtype=torch.bfloat16)]
    for out in bad_out:
        with pytest.raises(ValueError):
            attn_fwd(q, k, v, mask="causal", out=out)
    for lse in [torch.empty((1, 4, 131), dtype=torch.float32, device="cuda"),
                torch.empty((1, 4, 130), dtype=torch.bfloat16, device="cuda"),
                torch.empty((4, 130), dtype=torch.float32, device="cuda")]:
        with pytest.raises(ValueError):
            attn_fwd(q, k, v, mask="causal", lse=lse)


# ------------------------------------------------------------ full-size configs
#
# Each configuration runs once on the GPU, with the arguments and launch
# configuration the benchmark times, and every row of every head is compared
# with the oracle.  The oracle runs one (batch, head) slice per host thread;
# the document configuration runs through the per-document causal reduction
# (rows of document [a, b) are causal attention over keys [a, b) alone),
# plus a sample of rows through the full 32768-key rows.

_GPU = {}


def gpu_config(name):
    """The kernel's output for a named configuration, computed once per module."""
    if name not in _GPU:
        case = workloads.prefill_config(name)
        say(f"[case] {name} B={case['B']} Hq={case['Hq']} Hkv={case['Hkv']} N={case['Nq']} d={case['d']} "
            f"mask={case['mask']} W={case['window']}")
        q, k, v = dev(case["q"], case["dtype"]), dev(case["k"], case["dtype"]), dev(case["v"], case["dtype"])
        o, lse = attn_fwd(q, k, v, scale=case["scale"], mask=case["mask"], window=case["window"],
                          doc_offsets=doc_tensor(case))
        torch.cuda.synchronize()
        _GPU.clear()   # keep one configuration's inputs and outputs on the host at a time
        _GPU[name] = (case, host_f64(o), host_f64(lse))
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return _GPU[name]


def sample_rows(N, seed, extra=()):
    rng = np.random.default_rng(seed)
    base = {0, 1, 127, 128, N - 1, N - 2, N // 2}
    base.update(int(x) for x in extra if 0 <= x < N)
    base.update(rng.choice(N, size=min(N, 384), replace=False).tolist())
    return np.array(sorted(base))


@pytest.mark.slow
def test_config_causal_b4h16n2048_all_rows():
    case, og, lg = gpu_config("c2_causal_b4h16n2048")
    o_ref, l_ref = oracle_prefill_by_head(case, "c2")
    compare(og, lg, o_ref, l_ref, BF16_TOL, "c2 all rows")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["c3a_gqa_causal_n8192", "c3b_gqa_window1024_n8192"])
def test_config_gqa_n8192_all_rows(name):
    case, og, lg = gpu_config(name)
    o_ref, l_ref = oracle_prefill_by_head(case, name)
    compare(og, lg, o_ref, l_ref, BF16_TOL, f"{name} all {case['Nq']} rows of {case['Hq']} heads")


@pytest.mark.slow
def test_config_document_n32768_all_rows_per_document():
    case, og, lg = gpu_config("c4_document_n32768")
    o_ref, l_ref = oracle_document_by_parts(case, "c4")
    compare(og, lg, o_ref, l_ref, BF16_TOL, f"c4 all {case['Nq']} rows of {case['Hq']} heads (per document)")


@pytest.mark.slow
def test_config_document_n32768_sampled_full_rows():
    case, og, lg = gpu_config("c4_document_n32768")
    off = case["doc_offsets"]
    edges = list(off[:-1]) + list(off[1:] - 1) + list(off[1:-1] - 1) + list(off[1:-1] + 1)
    rows = sample_rows(case["Nq"], 2, extra=edges)
    o_ref, l_ref = oracle_prefill(case, rows=rows)
    compare(og[:, :, rows], lg[:, :, rows], o_ref, l_ref, BF16_TOL, f"c4 sampled {rows.size} full rows/head")
