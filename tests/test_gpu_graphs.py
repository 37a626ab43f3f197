"""The entry points under HIP graph capture.

Prefill, paged decode, chunked prefill and the backward (with learned sinks,
whose gradient is cleared by a kernel rather than a memset) are captured into
one graph with their outputs and workspaces allocated at capture.  The graph
is replayed several times; between replays the inputs are rewritten in place
and eager calls run on the same stream.  Every replay must match an eager call
on the same inputs: bit for bit, except the sink gradient, whose float atomics
may add in another order."""
import numpy as np
import pytest
import torch

import workloads
from exact_io_aware_fwd_amd import attn_bwd, attn_fwd, attn_paged_decode, attn_paged_prefill
from _gpu_helpers import dev, say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_calls():
    p = workloads.make_backward(1, 8, 2, 300, 300, 128, seed=111, mask="window", window=64)
    d = workloads.make_decode(4, 8, 2, 128, seq_lens=[5, 700, 1500, 33], max_seq_len=1500, seed=112,
                              tail_fill="nan")
    c = workloads.make_chunked_prefill(3, 8, 2, 128, chunks=[40, 1, 130], prefixes=[100, 7, 900], seed=113,
                                       tail_fill="nan")
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    q, k, v, do = dev(p["q"], "bf16"), dev(p["k"], "bf16"), dev(p["v"], "bf16"), dev(p["do"], "bf16")
    sinks = torch.tensor([0.5, -1.0, 2.0, 0.0, 1.0, -2.0, 0.3, 3.0], device="cuda")
    dq_, dk_, dv_ = dev(d["q"], "bf16"), dev(d["k_pages"], "bf16"), dev(d["v_pages"], "bf16")
    dbt, dsl = i32(d["block_table"]), i32(d["seq_lens"])
    cq, ck, cv = dev(c["q"], "bf16"), dev(c["k_pages"], "bf16"), dev(c["v_pages"], "bf16")
    cbt, csl, cqo = i32(c["block_table"]), i32(c["seq_lens"]), i32(c["q_offsets"])
    fkw = dict(scale=p["scale"], mask="window", window=64, sink_tokens=4, sink_logits=sinks)

    def step():
        o, lse = attn_fwd(q, k, v, **fkw)
        grads = attn_bwd(q, k, v, o, do, lse, **fkw)
        od, ld = attn_paged_decode(dq_, dk_, dv_, dbt, dsl, max_seq_len=d["max_seq_len"], scale=d["scale"],
                                   sink_logits=sinks)
        oc, lc = attn_paged_prefill(cq, ck, cv, cbt, csl, cqo, max_seq_len=c["max_seq_len"],
                                    max_q_len=c["max_q_len"], scale=c["scale"], mask="causal")
        return [o, lse, *grads, od, ld, oc, lc]

    say("[case] graph capture of prefill, backward, decode and chunked prefill")
    step()                                            # warm up (library load, first launches)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    torch.cuda.synchronize()
    names = ["o", "lse", "dq", "dk", "dv", "dsink", "decode o", "decode lse", "chunked o", "chunked lse"]
    gen = torch.Generator(device="cuda").manual_seed(114)
    for rep in range(4):
        if rep > 0:                                   # new inputs, written in place
            for t in (q, do, dq_, cq):
                t.copy_(torch.randn(t.shape, device="cuda", generator=gen).to(t.dtype))
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        want = step()                                 # eager, same stream, same inputs
        torch.cuda.synchronize()
        for name, a, b in zip(names, got, want):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from eager"
        say(f"[graph] replay {rep}: all outputs match the eager call")
