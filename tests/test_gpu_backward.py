"""Backward pass on the GPU against the fp64 oracle's gradients: dq, dk, dv
(and the learned sinks' gradient) after the GPU forward, over every mask kind,
GQA, ragged sizes, rows that see nothing, both sink forms, the score
modifications and both head dims (128, and 64 in the tests at the end).

Tolerance (no stated bound covers gradients; derived from the arithmetic):
P and dS enter their products rounded to bf16 (relative 2^-9 each) and D
uses the forward's bf16 output, so errors of a few tenths of a percent of the
gradient's scale are expected; the bound is 2e-2 relative Frobenius error
per tensor and 2e-2 x max|reference| on every element."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_io_aware_fwd_amd import attn_bwd, attn_fwd
from _gpu_helpers import dev, doc_tensor, host_f64, say

pytestmark = pytest.mark.gpu

REL_FRO = 2e-2
REL_MAX = 2e-2


def check_grad(got, want, label):
    err = np.abs(got - want)
    scale = float(np.abs(want).max()) if want.size else 0.0
    fro = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30))
    say(f"[grad] {label}: rel-fro {fro:.3e} max-abs {float(err.max()) if err.size else 0.0:.3e} (scale {scale:.3e})")
    assert np.all(np.isfinite(got)), f"{label}: non-finite gradient"
    if scale == 0.0:
        assert np.all(got == 0.0), f"{label}: gradient must be 0"
        return
    assert fro <= REL_FRO, f"{label}: relative Frobenius error {fro}"
    assert float(err.max()) <= REL_MAX * scale, f"{label}: max-abs {float(err.max())} > {REL_MAX} x {scale}"


def run_case(c, label, sink_tokens=0, sinks=None, softcap=0.0, slopes=None):
    say(f"[case] {label} B={c['B']} Hq={c['Hq']} Hkv={c['Hkv']} Nq={c['Nq']} Nk={c['Nk']} mask={c['mask']} "
        f"window={c['window']} sink_tokens={sink_tokens} sinks={'yes' if sinks is not None else 'no'} "
        f"softcap={softcap} alibi={'yes' if slopes is not None else 'no'}")
    q, k, v, do = dev(c["q"], "bf16"), dev(c["k"], "bf16"), dev(c["v"], "bf16"), dev(c["do"], "bf16")
    sl = None if sinks is None else torch.from_numpy(sinks).cuda()
    kw = dict(scale=c["scale"], mask=c["mask"], window=c["window"], doc_offsets=doc_tensor(c),
              sink_tokens=sink_tokens, sink_logits=sl, softcap=softcap,
              alibi_slopes=None if slopes is None else torch.from_numpy(slopes).cuda())
    o, lse = attn_fwd(q, k, v, **kw)
    dq, dk, dv, ds = attn_bwd(q, k, v, o, do, lse, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(oracle.to_f64(c["q"], "bf16"), oracle.to_f64(c["k"], "bf16"),
                                    oracle.to_f64(c["v"], "bf16"), oracle.to_f64(c["do"], "bf16"), c["scale"],
                                    c["mask"], c["window"], c["doc_offsets"], sink_tokens,
                                    None if sinks is None else sinks.astype(np.float64), softcap=softcap,
                                    alibi_slopes=None if slopes is None else slopes.astype(np.float64))
    grads = []
    for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        grads.append(host_f64(got))
        check_grad(grads[-1], want, f"{label} {name}")
    if sinks is not None:
        check_grad(host_f64(ds), ref[3], f"{label} dsink")
    return grads


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_bitwise_identical_run_to_run(dtype):
    """Every gradient, the sink's included, is the same bit for bit on every
    call: no pass uses atomics (the sink gradient is a fixed-order reduction)."""
    c = workloads.make_backward(2, 8, 2, 700, 700, 128, dtype=dtype, seed=75, mask="window", window=200)
    q, k, v, do = (dev(c[x], dtype) for x in ("q", "k", "v", "do"))
    sinks = torch.from_numpy(np.random.default_rng(76).normal(0.0, 1.5, 8).astype(np.float32)).cuda()
    kw = dict(scale=c["scale"], mask="window", window=200, sink_tokens=4, sink_logits=sinks)
    o, lse = attn_fwd(q, k, v, **kw)
    first = attn_bwd(q, k, v, o, do, lse, **kw)
    for _ in range(3):
        again = attn_bwd(q, k, v, o, do, lse, **kw)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dsink"), first, again):
            assert torch.equal(a, b), f"{dtype} {name} differs between calls"
    say(f"[grad] {dtype}: four calls bit-identical, dsink {first[3].tolist()}")


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 100), ("document", 0)])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4)])
def test_backward_masks(mask, window, Hq, Hkv):
    c = workloads.make_backward(1, Hq, Hkv, 600, 600, 128, seed=71, mask=mask, window=window, doc_min=80,
                                doc_max=300)
    run_case(c, f"bwd {mask} Hq{Hq}Hkv{Hkv}")


@pytest.mark.parametrize("Nq,Nk", [(300, 200), (129, 500), (65, 65), (1, 130)])
def test_backward_ragged_and_aligned(Nq, Nk):
    # causal, bottom-right: Nq > Nk leaves the first rows with no key
    c = workloads.make_backward(2, 4, 2, Nq, Nk, 128, seed=73, mask="causal")
    run_case(c, f"bwd causal {Nq}x{Nk}")


@pytest.mark.parametrize("d", [128, 64])
def test_backward_keys_no_row_sees(d):
    # window 50, bottom-right aligned: the 100 rows see only keys 851..999,
    # so the first key blocks get no query tile at all (an empty loop) and
    # their dK and dV rows must come out exactly zero
    c = workloads.make_backward(1, 4, 2, 100, 1000, d, seed=95, mask="window", window=50)
    _, dk, dv = run_case(c, f"bwd window50 100x1000 d{d}")
    assert np.all(dk[:, :, :851] == 0.0) and np.all(dv[:, :, :851] == 0.0), "unseen keys must get zero gradients"
    assert np.any(dk[:, :, 851:] != 0.0) and np.any(dv[:, :, 851:] != 0.0)


@pytest.mark.parametrize("sink_tokens,with_logits", [(4, True), (70, False), (0, True)])
def test_backward_sinks(sink_tokens, with_logits):
    c = workloads.make_backward(1, 8, 2, 500, 500, 128, seed=75, mask="window", window=96)
    sinks = None
    if with_logits:
        sinks = np.random.default_rng(76).normal(0.0, 2.0, 8).astype(np.float32)
    run_case(c, f"bwd window96 sinks{sink_tokens}", sink_tokens, sinks)


def test_backward_larger_causal():
    c = workloads.make_backward(1, 8, 2, 2048, 2048, 128, seed=77, mask="causal")
    run_case(c, "bwd causal 2048 GQA")


def alibi_slopes(Hq):
    return np.array([2.0 ** (-8.0 * (h + 1) / Hq) for h in range(Hq)], dtype=np.float32)


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 100), ("document", 0)])
@pytest.mark.parametrize("softcap,alibi", [(2.0, False), (0.0, True), (3.0, True)])
def test_backward_score_mods(mask, window, softcap, alibi):
    # scale 3/sqrt(d): scores of a few units, so the caps bend most of them
    c = workloads.make_backward(1, 8, 2, 500, 500, 128, seed=77, mask=mask, window=window, doc_min=80,
                                doc_max=300, scale=3.0 / np.sqrt(128))
    run_case(c, f"bwd mods {mask} cap{softcap} alibi{alibi}", softcap=softcap,
             slopes=alibi_slopes(8) if alibi else None)


def test_backward_score_mods_ragged_with_sinks():
    # Nq > Nk: the first rows see no key; window with sink tokens and learned sinks
    c = workloads.make_backward(2, 4, 2, 300, 200, 128, seed=79, mask="causal", scale=0.2)
    run_case(c, "bwd mods causal 300x200", softcap=1.5, slopes=alibi_slopes(4))
    c = workloads.make_backward(1, 8, 2, 500, 500, 128, seed=81, mask="window", window=96, scale=0.2)
    sinks = np.random.default_rng(82).normal(0.0, 2.0, 8).astype(np.float32)
    run_case(c, "bwd mods window96 sinks", 4, sinks, softcap=2.5, slopes=alibi_slopes(8))


@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 70), ("document", 0)])
def test_backward_d64_masks(mask, window):
    c = workloads.make_backward(1, 8, 2, 520, 520, 64, seed=83, mask=mask, window=window, doc_min=60, doc_max=250)
    run_case(c, f"bwd d64 {mask}")


@pytest.mark.parametrize("Nq,Nk", [(300, 200), (65, 65), (1, 130), (129, 500)])
def test_backward_d64_ragged(Nq, Nk):
    c = workloads.make_backward(2, 4, 4, Nq, Nk, 64, seed=85, mask="causal")
    run_case(c, f"bwd d64 causal {Nq}x{Nk}")


def test_backward_d64_sinks_and_mods():
    c = workloads.make_backward(1, 8, 2, 500, 500, 64, seed=87, mask="window", window=96, scale=0.25)
    sinks = np.random.default_rng(88).normal(0.0, 2.0, 8).astype(np.float32)
    run_case(c, "bwd d64 window96 sinks", 4, sinks)
    run_case(c, "bwd d64 window96 sinks + mods", 4, sinks, softcap=2.0, slopes=alibi_slopes(8))


def test_backward_c2_full_size_sampled_heads():
    """The backward of the 2048-token causal MHA workload (B 4, H 16, d 128)
    in the launch configuration the benchmark times; the oracle on three
    sampled (batch, head) pairs.  With one query head per KV head a head's
    gradients depend on that head alone, so each sample is exact."""
    c = workloads.make_backward(4, 16, 16, 2048, 2048, 128, seed=0, mask="causal")
    say("[case] backward of c2 at full size, sampled heads")
    q, k, v, do = dev(c["q"], "bf16"), dev(c["k"], "bf16"), dev(c["v"], "bf16"), dev(c["do"], "bf16")
    o, lse = attn_fwd(q, k, v, scale=c["scale"], mask="causal")
    dq, dk, dv, _ = attn_bwd(q, k, v, o, do, lse, scale=c["scale"], mask="causal")
    torch.cuda.synchronize()
    f64 = lambda a, b, h: oracle.to_f64(a[b:b + 1, h:h + 1], "bf16")
    for b, h in [(0, 0), (1, 7), (3, 15)]:
        ref = oracle.attention_backward(f64(c["q"], b, h), f64(c["k"], b, h), f64(c["v"], b, h), f64(c["do"], b, h),
                                        c["scale"], "causal")
        for name, got, want in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
            check_grad(host_f64(got[b:b + 1, h:h + 1]), want, f"c2 b{b} h{h} {name}")


# fp32 checking path: inputs, outputs and gradients in float32.  Bound derived
# for fp32 accumulation over a few hundred terms (about 1e-6 relative in
# practice): relative Frobenius 2e-5, every element within 1e-4 x max|reference|.
def run_case_f32(c, label, sink_tokens=0, sinks=None, softcap=0.0, slopes=None):
    say(f"[case] {label} fp32 Nq={c['Nq']} Nk={c['Nk']} d={c['d']} mask={c['mask']} window={c['window']}")
    q, k, v, do = (dev(c[x], "f32") for x in ("q", "k", "v", "do"))
    kw = dict(scale=c["scale"], mask=c["mask"], window=c["window"], doc_offsets=doc_tensor(c),
              sink_tokens=sink_tokens, sink_logits=None if sinks is None else torch.from_numpy(sinks).cuda(),
              softcap=softcap, alibi_slopes=None if slopes is None else torch.from_numpy(slopes).cuda())
    o, lse = attn_fwd(q, k, v, **kw)
    dq, dk, dv, ds = attn_bwd(q, k, v, o, do, lse, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(*(oracle.to_f64(c[x], "f32") for x in ("q", "k", "v", "do")), c["scale"],
                                    c["mask"], c["window"], c["doc_offsets"], sink_tokens,
                                    None if sinks is None else sinks.astype(np.float64), softcap=softcap,
                                    alibi_slopes=None if slopes is None else slopes.astype(np.float64))
    got = [host_f64(dq), host_f64(dk), host_f64(dv)] + ([host_f64(ds)] if sinks is not None else [])
    for name, g, w in zip(("dq", "dk", "dv", "dsink"), got, ref):
        fro = float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-30))
        mx = float(np.abs(g - w).max())
        say(f"[grad] {label} fp32 {name}: rel-fro {fro:.3e} max-abs {mx:.3e}")
        assert np.all(np.isfinite(g)) and fro <= 2e-5 and mx <= 1e-4 * float(np.abs(w).max()), f"{label} {name}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 50), ("document", 0)])
def test_backward_f32(d, mask, window):
    c = workloads.make_backward(1, 4, 2, 200, 200, d, dtype="f32", seed=89, mask=mask, window=window,
                                doc_min=30, doc_max=90)
    run_case_f32(c, f"bwd {mask} d{d}")


def test_backward_f32_ragged_sinks_and_mods():
    c = workloads.make_backward(2, 4, 2, 150, 100, 128, dtype="f32", seed=91, mask="causal")
    run_case_f32(c, "bwd causal 150x100")          # Nq > Nk: the first rows see no key
    c = workloads.make_backward(1, 4, 2, 220, 220, 64, dtype="f32", seed=93, mask="window", window=40, scale=0.3)
    sinks = np.array([0.5, -1.0, 2.0, 0.0], dtype=np.float32)
    run_case_f32(c, "bwd window sinks + mods", 3, sinks, softcap=2.0, slopes=alibi_slopes(4))
