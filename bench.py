#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one causal bf16 prefill (B=4, Hq=Hkv=16, N=2048, d=128, the
headline workload) followed by one paged decode (64 sequences, Hq=32, Hkv=8,
d=128, context lengths uniform in [1024, 32768], 16-token pages, seeded
random page placement).  Inputs are seeded synthetic data, generated on the
host, copied once and resident in HBM before any timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Runs W untimed steps, then times K steps between two synchronisations
(`ms_per_step`).  Every workload ("leg") is then timed on its own: 10 warm-up
calls, then at least 100 calls, each between two HIP events on the launch
stream; the median, p10 and p90 of the per-call times are reported.  The legs
are the five prefill workloads' four bf16 ones (C2 causal 4x16x2048, C3a GQA
causal 8192, C3b GQA window-1024 8192, C4 document 32768), the paged decode
(C5), the chunked prefill over the paged cache (C6) and the backward of C2.
Beside the decode leg, a standalone streaming-read probe (_build/hbm_read_probe,
built with the library) reads the same number of bytes once, as the practical
read rate next to the published HBM peak (`--no-read-ceiling` skips it).

Prints ONE JSON line.  `value` is the C2 prefill's algorithmic TFLOP/s
(4·d·B·Hq·visible pairs per call ÷ the median call time); the other legs are
under `legs`.  `cpu_baseline` is the fp64 numpy oracle, as it is, timed on
this host's cores: C1 whole (its seconds are the headline "oracle in
seconds"), C2 whole, and bounded samples of C3a, C3b, C4 and C5 with the
extrapolation to the whole workload labelled as such.

    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR

turns two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
`bench.py --pmc-pass` into profiles/hbm_traffic.json.

    python bench.py --summarize-clock DIR

turns one `rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE` run of
`bench.py --pmc-pass` into per-launch GPU cycles, the shader clock the
kernel actually ran at (cycles / duration) and, for the forward kernels,
the MFMA utilisation in cycles: profiles/sclk_per_workload.json.

The --pmc-pass launches every workload a fixed number of times in the order
of PMC_PLAN, so a dispatch's workload follows from its kernel and its rank
among that kernel's dispatches.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6     # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0         # HBM3E
PREFILL_CONFIG = "c2_causal_b4h16n2048"
DECODE_CONFIG = "c5_paged_decode_64"
CHUNKED_CONFIG = "c6_chunked_prefill_16"
PREFILL_LEGS = {"c2": "c2_causal_b4h16n2048", "c3a": "c3a_gqa_causal_n8192",
                "c3b": "c3b_gqa_window1024_n8192", "c4": "c4_document_n32768"}
# kernels each leg launches, once per call, in launch order
LEG_KERNELS = {
    "c2": ["prefill_bf16_kernel<128, false>"], "c3a": ["prefill_bf16_kernel<128, false>"],
    "c3b": ["prefill_bf16_k32_kernel<false>"], "c4": ["prefill_bf16_k32_kernel<false>"],
    "c5": ["decode_split_kernel<128, false>", "decode_combine_kernel<128>"],
    "c6": ["paged_prefill_swz_kernel<false>"],
    "bwd_c2": ["bwd_dq_kernel", "bwd_dkdv2_kernel"],
}
LEG_WORKLOAD = {"c2": PREFILL_LEGS["c2"], "c3a": PREFILL_LEGS["c3a"], "c3b": PREFILL_LEGS["c3b"],
                "c4": PREFILL_LEGS["c4"], "c5": DECODE_CONFIG, "c6": CHUNKED_CONFIG,
                "bwd_c2": "backward of " + PREFILL_CONFIG}
# the --pmc-pass: (leg, calls), in this order
PMC_PLAN = [("c2", 3), ("c3a", 2), ("c3b", 2), ("c4", 2), ("c5", 3), ("c6", 2), ("bwd_c2", 2)]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CLOCK_FILE = os.path.join(ROOT, "profiles", "sclk_per_workload.json")
NUM_XCD = 8                   # GRBM_GUI_ACTIVE is counted once per accelerator die
MFMA_FLOP_PER_CLK = 256 * 4096  # dense bf16 MFMA, whole GPU, per shader clock
CSRC = os.path.join(ROOT, "exact_io_aware_fwd_amd", "csrc")
COPY_BYTES = 1 << 30          # known-size copy used to calibrate the HBM byte counters
LEG_CALLS = 100               # timed calls per leg (at least)
LEG_WARMUP = 10


def read_ceiling(nbytes: int):
    """The practical HBM read rate beside the published peak: the standalone
    streaming-read probe (built with the library into _build/) reads a buffer
    of the decode call's byte count linearly and as 4 KiB pages in a random
    order; the best median of each pattern over a small sweep of grids, loads
    in flight and load kinds.  None when the probe is not built or fails."""
    exe = os.path.join(ROOT, "_build", "hbm_read_probe")
    if not os.path.exists(exe):
        return None
    try:
        r = subprocess.run([exe, str(int(nbytes))], capture_output=True, text=True, timeout=120)
    except subprocess.TimeoutExpired:
        log("read-ceiling probe timed out")
        return None
    if r.returncode != 0:
        log(f"read-ceiling probe failed: {r.stderr.strip()[-200:]}")
        return None
    lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
    return json.loads(lines[-1]) if lines else None


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------- work accounting

def visible_pairs(Nq: int, Nk: int, mask: str, window: int = 0, doc_offsets=None) -> int:
    """Number of (query, key) pairs a mask lets through, per (batch, head)."""
    i = np.arange(Nq, dtype=np.int64)
    pos = i + (Nk - Nq)
    if mask == "none":
        return Nq * Nk
    hi = np.minimum(pos, Nk - 1)
    if mask == "causal":
        lo = np.zeros_like(pos)
    elif mask == "window":
        lo = np.maximum(pos - window + 1, 0)
    elif mask == "document":
        off = np.asarray(doc_offsets, dtype=np.int64)
        lo = off[np.clip(np.searchsorted(off, np.maximum(pos, 0), side="right") - 1, 0, len(off) - 2)]
    else:
        raise ValueError(mask)
    cnt = np.where(pos >= 0, hi - lo + 1, 0)
    return int(np.clip(cnt, 0, None).sum())


def prefill_flops(c: dict) -> int:
    return 4 * c["d"] * c["B"] * c["Hq"] * visible_pairs(c["Nq"], c["Nk"], c["mask"], c["window"], c["doc_offsets"])


def chunked_visible_pairs(c: dict) -> int:
    """Visible (query, key) pairs of a chunked prefill, per query head: chunk s
    is a problem with Nq = chunk length and Nk = cached length (bottom-right)."""
    offs = np.asarray(c["q_offsets"], dtype=np.int64)
    return sum(visible_pairs(int(offs[s + 1] - offs[s]), int(c["seq_lens"][s]), c["mask"], c["window"])
               for s in range(c["num_seqs"]))


def chunked_flops(c: dict) -> int:
    return 4 * c["d"] * c["Hq"] * chunked_visible_pairs(c)


def prefill_bytes(c: dict) -> int:
    el = 2 if c["dtype"] == "bf16" else 4
    q = c["B"] * c["Hq"] * c["Nq"] * c["d"] * el
    kv = 2 * c["B"] * c["Hkv"] * c["Nk"] * c["d"] * el
    return q + kv + q + c["B"] * c["Hq"] * c["Nq"] * 4


def decode_bytes(c: dict) -> int:
    """HBM bytes a paged decode must move: the cache it reads, q, o, lse and the index data."""
    lens = c["seq_lens"].astype(np.int64)
    S, Hq, Hkv, d = c["num_seqs"], c["Hq"], c["Hkv"], c["d"]
    kv = int(lens.sum()) * Hkv * d * 2 * 2
    pages = int((-(-lens // c["page_size"])).sum())
    return kv + 2 * S * Hq * d * 2 + S * Hq * 4 + pages * 4 + S * 4


def source_digest() -> str:
    """SHA-256 over the kernel sources' names and bytes (files only: a cache
    directory beside them does not count)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        if not os.path.isfile(p):
            continue
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()


def measured_traffic(leg: str):
    """HBM bytes per call of a leg (all its kernels) from the committed counter
    summary, or None when there is none or the kernel sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    t = json.load(open(TRAFFIC_FILE))
    if t.get("source_sha256") != source_digest():
        return None
    total = 0.0
    for kern in LEG_KERNELS[leg]:
        k = t.get("legs", {}).get(leg, {}).get(kern)
        if not k:
            return None
        total += k["fetch_bytes"] + k["write_bytes"]
    return int(total)


def percentiles(us) -> dict:
    us = np.asarray(us, dtype=np.float64)
    return {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
            "p90": round(float(np.percentile(us, 90)), 2), "mean": round(float(np.mean(us)), 2), "calls": int(us.size)}


# -------------------------------------------------------------- CPU baseline

def cpu_baseline(hosts: dict) -> dict:
    """The fp64 oracle, as it is, on this host's cores (BLAS threads = the
    cores this process may run on).  C1 and C2 run whole; C3a, C3b, C4 and C5
    run a bounded sample whose seconds are scaled to the whole workload (rows
    are independent, so the oracle's time is linear in them) and labelled as
    an extrapolation.  `value` is the C2 throughput in the metric's unit.
    hosts: the legs' host-side inputs already generated ({leg: config dict});
    the others are generated here."""
    import oracle
    from threadpoolctl import threadpool_limits

    cores = len(os.sched_getaffinity(0))
    per = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def prefill_slices(c, heads, rows=None):
        g = c["Hq"] // c["Hkv"]
        for b, h in heads:
            hk = h // g
            q = oracle.to_f64(c["q"][b:b + 1, h:h + 1], c["dtype"])
            k = oracle.to_f64(c["k"][b:b + 1, hk:hk + 1], c["dtype"])
            v = oracle.to_f64(c["v"][b:b + 1, hk:hk + 1], c["dtype"])
            oracle.attention(q, k, v, c["scale"], c["mask"], c["window"], c["doc_offsets"], rows=rows)

    with threadpool_limits(limits=cores):
        c1 = workloads.prefill_config("c1_f32_single_head")
        sec = min(timed(lambda: prefill_slices(c1, [(0, 0)])) for _ in range(3))
        per["c1"] = {"seconds": round(sec, 4), "sample": "whole (best of 3)", "gflop": round(prefill_flops(c1) / 1e9, 4)}
        log(f"oracle c1: {sec:.4f} s")

        get = lambda leg: hosts.get(leg) or workloads.prefill_config(PREFILL_LEGS[leg])
        c2 = get("c2")
        heads = [(b, h) for b in range(c2["B"]) for h in range(c2["Hq"])]
        sec2 = timed(lambda: prefill_slices(c2, heads))
        f2 = prefill_flops(c2)
        per["c2"] = {"seconds": round(sec2, 3), "sample": "whole", "tflops": round(f2 / sec2 / 1e12, 6)}
        log(f"oracle c2: {sec2:.2f} s")

        for leg, nheads in (("c3a", 2), ("c3b", 2)):
            c = get(leg)
            sec = timed(lambda: prefill_slices(c, [(0, h) for h in range(nheads)]))
            per[leg] = {"seconds_sample": round(sec, 3), "sample": f"{nheads} of {c['Hq']} heads, all rows",
                        "seconds_extrapolated": round(sec * c["Hq"] / nheads, 1)}
            log(f"oracle {leg}: {sec:.2f} s for {nheads} heads")
            del c

        c4 = get("c4")
        rows = np.unique(np.concatenate([c4["doc_offsets"][:-1], c4["doc_offsets"][1:] - 1,
                                         np.random.default_rng(4).choice(c4["Nq"], 256, replace=False)]))
        sec = timed(lambda: prefill_slices(c4, [(0, 0)], rows=rows))
        per["c4"] = {"seconds_sample": round(sec, 3),
                     "sample": f"{rows.size} full rows of 1 of {c4['Hq']} heads (every document's first and last "
                               f"row, 256 random)",
                     "seconds_extrapolated": round(sec * c4["Nq"] * c4["Hq"] / rows.size, 1)}
        log(f"oracle c4: {sec:.2f} s for {rows.size} rows")
        del c4

        c5 = hosts.get("c5") or workloads.decode_config(DECODE_CONFIG)
        seqs = list(range(8))
        sec = timed(lambda: oracle.paged_decode(c5["q"], c5["k_pages"], c5["v_pages"], c5["block_table"],
                                                 c5["seq_lens"], c5["scale"], seqs=seqs, dtype="bf16"))
        frac = float(c5["seq_lens"][seqs].sum()) / float(c5["seq_lens"].sum())
        per["c5"] = {"seconds_sample": round(sec, 3),
                     "sample": f"{len(seqs)} of {c5['num_seqs']} sequences ({100 * frac:.1f} % of the cached tokens)",
                     "seconds_extrapolated": round(sec / frac, 1)}
        log(f"oracle c5: {sec:.2f} s for {len(seqs)} sequences")
        del c5

    return {"value": per["c2"]["tflops"], "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{PREFILL_LEGS['c2']}: all 64 (batch, head) slices, all 2048 rows, {sec2:.2f} s fp64 numpy; "
                      f"per_config holds C1 (whole), C3a, C3b, C4, C5 (samples)",
            "c1_seconds": per["c1"]["seconds"], "per_config": per}


# ------------------------------------------------------------------- GPU run

def to_dev(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def time_calls(fn, calls: int, warmup: int):
    """Per-call microseconds of fn: warm-up calls, then each call between two
    HIP events recorded on torch's current stream (the launch stream)."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


class Prefill:
    """One prefill workload resident on the GPU."""

    def __init__(self, name: str):
        import torch
        self.name = name
        self.c = workloads.prefill_config(name)
        c = self.c
        self.q, self.k, self.v = to_dev(c["q"]), to_dev(c["k"]), to_dev(c["v"])
        self.doc = torch.from_numpy(c["doc_offsets"]).cuda() if c["doc_offsets"] is not None else None
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((c["B"], c["Hq"], c["Nq"]), dtype=torch.float32, device="cuda")
        self.flops = prefill_flops(c)

    def __call__(self):
        from exact_io_aware_fwd_amd import attn_fwd
        c = self.c
        attn_fwd(self.q, self.k, self.v, scale=c["scale"], mask=c["mask"], window=c["window"], doc_offsets=self.doc,
                 out=self.o, lse=self.lse)

    def describe(self) -> str:
        c = self.c
        m = c["mask"] + (f" {c['window']}" if c["mask"] == "window" else "")
        return f"{self.name} (B{c['B']} Hq{c['Hq']} Hkv{c['Hkv']} N{c['Nq']} d{c['d']} {m})"


class Decode:
    def __init__(self):
        import torch
        from exact_io_aware_fwd_amd import attn_paged_decode_workspace_size
        self.c = c = workloads.decode_config(DECODE_CONFIG)
        self.q, self.kp, self.vp = to_dev(c["q"]), to_dev(c["k_pages"]), to_dev(c["v_pages"])
        self.bt = torch.from_numpy(c["block_table"]).cuda()
        self.sl = torch.from_numpy(c["seq_lens"]).cuda()
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((c["num_seqs"], c["Hq"]), dtype=torch.float32, device="cuda")
        self.ws = torch.empty(attn_paged_decode_workspace_size(c["num_seqs"], c["Hq"], c["d"], c["max_seq_len"]),
                              dtype=torch.uint8, device="cuda")
        self.bytes = decode_bytes(c)

    def __call__(self):
        from exact_io_aware_fwd_amd import attn_paged_decode
        c = self.c
        attn_paged_decode(self.q, self.kp, self.vp, self.bt, self.sl, max_seq_len=c["max_seq_len"], scale=c["scale"],
                          workspace=self.ws, out=self.o, lse=self.lse)


class Chunked:
    def __init__(self):
        import torch
        self.c = c = workloads.chunked_config(CHUNKED_CONFIG)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        self.q, self.kp, self.vp = to_dev(c["q"]), to_dev(c["k_pages"]), to_dev(c["v_pages"])
        self.bt, self.sl, self.qo = i32(c["block_table"]), i32(c["seq_lens"]), i32(c["q_offsets"])
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(self.q.shape[:2], dtype=torch.float32, device="cuda")
        self.flops = chunked_flops(c)

    def __call__(self):
        from exact_io_aware_fwd_amd import attn_paged_prefill
        c = self.c
        attn_paged_prefill(self.q, self.kp, self.vp, self.bt, self.sl, self.qo, max_seq_len=c["max_seq_len"],
                           max_q_len=c["max_q_len"], scale=c["scale"], mask=c["mask"], out=self.o, lse=self.lse)

    def describe(self) -> str:
        c = self.c
        return (f"{CHUNKED_CONFIG} ({c['num_seqs']} seqs, Hq{c['Hq']} Hkv{c['Hkv']} d{c['d']}, "
                f"{int(c['q_offsets'][-1])} chunk tokens over {int(c['seq_lens'].sum())} cached, causal)")


class Backward:
    """Backward of the C2 prefill from that prefill's own o and lse."""

    def __init__(self, pre: Prefill):
        import torch
        from exact_io_aware_fwd_amd import attn_bwd_workspace_size
        self.p = pre
        c = pre.c
        self.do = to_dev(workloads.gen._draw(0, 5, (c["B"], c["Hq"], c["Nq"], c["d"]), "bf16"))
        self.ws = torch.empty(attn_bwd_workspace_size(c["B"], c["Hq"], c["Nq"]), dtype=torch.uint8, device="cuda")
        self.flops = backward_flops(c)

    def __call__(self):
        from exact_io_aware_fwd_amd import attn_bwd
        p, c = self.p, self.p.c
        attn_bwd(p.q, p.k, p.v, p.o, self.do, p.lse, scale=c["scale"], mask=c["mask"], window=c["window"],
                 doc_offsets=p.doc, workspace=self.ws)


def backward_flops(c: dict) -> int:
    """The backward's five products per visible pair (recomputed scores, dP,
    dV, dK, dQ), 2 d flops each."""
    return 10 * c["d"] * c["B"] * c["Hq"] * visible_pairs(c["Nq"], c["Nk"], c["mask"], c["window"], c["doc_offsets"])


def flops_leg(name: str, flops: int, us: list, kernel: str, workload: str) -> dict:
    st = percentiles(us)
    tf = flops / (st["median"] * 1e-6) / 1e12
    log(f"{name}: median {st['median']:.1f} us (p10 {st['p10']:.1f}, p90 {st['p90']:.1f}) -> {tf:.1f} TFLOP/s "
        f"({100 * tf / PEAK_BF16_TFLOPS:.1f} % of peak)")
    return {"workload": workload, "kernel": kernel, "flop_per_call": flops, "us": st, "tflops": round(tf, 2),
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(name)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--calls", type=int, default=LEG_CALLS, help="timed calls per leg (at least 100 kept)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true", help="skip the streaming-read probe beside the decode leg")
    ap.add_argument("--legs", default="c3a,c3b,c4,c6,bwd_c2",
                    help="legs timed beside C2 and C5 (comma list of c3a,c3b,c4,c6,bwd_c2; empty for none)")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="short run for counter collection: one known-size copy, then PMC_PLAN's launches")
    ap.add_argument("--repeat", type=int, default=1, help="--pmc-pass: run the plan's calls this many times over")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="every counter of one or more --pmc runs of --pmc-pass, per workload: profiles/sq_counters.json")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="per-workload kernel durations from a --kernel-trace run of --pmc-pass")
    ap.add_argument("--summarize-clock", metavar="DIR")
    args = ap.parse_args()

    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc)
    if args.summarize_clock:
        return summarize_clock(args.summarize_clock)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the library has no multi-GPU path "
                                   "(--gpus must be 1)"}))
        return 2

    import torch

    torch.cuda.set_device(0)
    if args.pmc_pass:
        return pmc_pass(max(1, args.repeat))

    calls = max(LEG_CALLS, args.calls)
    hosts = {}   # host-side inputs of the legs, reused by the CPU baseline
    log(f"generating inputs ({PREFILL_LEGS['c2']}, {DECODE_CONFIG})")
    pre = Prefill(PREFILL_LEGS["c2"])
    dec = Decode()
    hosts["c2"], hosts["c5"] = pre.c, dec.c
    torch.cuda.synchronize()
    log("inputs resident on the GPU")

    # ---- the step loop: W untimed steps, K timed steps between two synchronisations
    K, W = args.steps, args.warmup
    for _ in range(W):
        pre()
        dec()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    for _ in range(K):
        pre()
        dec()
    end.record()
    torch.cuda.synchronize()
    step_ms = start.elapsed_time(end) / K
    log(f"timed {K} steps: {step_ms:.3f} ms/step (wall {time.perf_counter() - wall0:.2f} s)")

    # ---- per-call legs
    legs = {}
    legs["c2"] = flops_leg("c2", pre.flops, time_calls(pre, calls, LEG_WARMUP), LEG_KERNELS["c2"][0], pre.describe())
    d_st = percentiles(time_calls(dec, calls, LEG_WARMUP))
    gbs = dec.bytes / (d_st["median"] * 1e-6) / 1e9
    log(f"c5: median {d_st['median']:.1f} us (p10 {d_st['p10']:.1f}, p90 {d_st['p90']:.1f}) -> {gbs:.1f} GB/s")
    legs["c5"] = {"workload": f"{DECODE_CONFIG} (64 seqs, Hq32 Hkv8 d128, 16-token pages, "
                              f"{int(dec.c['seq_lens'].sum())} cached tokens)",
                  "kernel": " + ".join(LEG_KERNELS["c5"]) + " (one call)", "bytes_per_call": dec.bytes, "us": d_st,
                  "gbs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("c5")}
    ceiling = None if args.no_read_ceiling else read_ceiling(dec.bytes)
    if ceiling is not None:
        lin, pg = ceiling["linear"], ceiling["pages"]
        log(f"read ceiling over {ceiling['bytes']} bytes: linear {lin['median_gbs']:.1f} GB/s, 4 KiB pages in "
            f"random order {pg['median_gbs']:.1f} GB/s (decode at {gbs / pg['median_gbs']:.3f} of the latter)")
        legs["c5"]["read_ceiling"] = {
            "pages_gbs": pg["median_gbs"], "linear_gbs": lin["median_gbs"],
            "decode_frac_of_pages": round(gbs / pg["median_gbs"], 4),
            "decode_frac_of_linear": round(gbs / lin["median_gbs"], 4),
            "probe": "_build/hbm_read_probe: the same byte count read once with 16-byte loads, linearly and as "
                     "4 KiB pages in a seeded random order; best median of each over grids, loads in flight and "
                     f"load kinds (pages: {pg['grid']} workgroups, {pg['pages_in_flight_per_wave']} pages in flight "
                     f"per wave, nontemporal {pg['nontemporal']}; linear: {lin['grid']} workgroups, "
                     f"{lin['loads_in_flight_per_lane']} loads in flight per lane, nontemporal {lin['nontemporal']})"}
    extra = [x for x in args.legs.split(",") if x]
    if "bwd_c2" in extra:
        bwd = Backward(pre)
        legs["bwd_c2"] = flops_leg("bwd_c2", bwd.flops, time_calls(bwd, calls, LEG_WARMUP),
                                   " + ".join(LEG_KERNELS["bwd_c2"]) + " (one call)", "backward of " + pre.describe())
        del bwd
    del dec
    torch.cuda.empty_cache()
    for leg in ("c3a", "c3b", "c4"):
        if leg in extra:
            log(f"generating inputs ({PREFILL_LEGS[leg]})")
            x = Prefill(PREFILL_LEGS[leg])
            legs[leg] = flops_leg(leg, x.flops, time_calls(x, calls, LEG_WARMUP), LEG_KERNELS[leg][0], x.describe())
            hosts[leg] = x.c
            del x
            torch.cuda.empty_cache()
    if "c6" in extra:
        log(f"generating inputs ({CHUNKED_CONFIG})")
        x = Chunked()
        legs["c6"] = flops_leg("c6", x.flops, time_calls(x, calls, LEG_WARMUP), LEG_KERNELS["c6"][0], x.describe())
        del x
        torch.cuda.empty_cache()

    c2 = legs["c2"]
    result = {
        "metric": "attn fwd TFLOP/s (% bf16 MFMA peak) causal prefill; paged decode HBM GB/s",
        "value": c2["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{pre.describe()} + {legs['c5']['workload']}",
            "prefill_flop_per_call": pre.flops,
            "prefill_us_median": c2["us"]["median"],
            "decode_bytes_per_call": legs["c5"]["bytes_per_call"],
            "decode_us_median": legs["c5"]["us"]["median"],
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100 * c2["frac"], 2),
        "roofline": {
            "bound": "mfma", "achieved": c2["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": c2["frac"], "traffic": c2["traffic"], "kernel": c2["kernel"],
            "algorithmic_bytes": prefill_bytes(pre.c), "timing": "median of per-call HIP events",
        },
        "decode": {
            "value": legs["c5"]["gbs"], "unit": "GB/s", "pct_of_peak": round(100 * legs["c5"]["frac"], 2),
            "roofline": {"bound": "hbm", "achieved": legs["c5"]["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": legs["c5"]["frac"], "traffic": legs["c5"]["traffic"], "kernel": legs["c5"]["kernel"]},
            "read_ceiling": legs["c5"].get("read_ceiling"),
        },
        "legs": legs,
    }
    del pre
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on host cores")
        result["cpu_baseline"] = cpu_baseline(hosts)
    print(json.dumps(result), flush=True)
    return 0


def pmc_pass(repeat: int = 1) -> int:
    """One known-size device copy (the byte-counter calibration), then every
    leg's calls in PMC_PLAN order, each count times `repeat` (no other launch
    of these kernels)."""
    import torch

    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    c2 = None
    for leg, n in PMC_PLAN:
        log(f"pmc pass: {leg} x {n}")
        if leg in PREFILL_LEGS:
            x = Prefill(PREFILL_LEGS[leg])
            if leg == "c2":
                c2 = x
        elif leg == "c5":
            x = Decode()
        elif leg == "c6":
            x = Chunked()
        else:
            x = Backward(c2)
        torch.cuda.synchronize()
        for _ in range(n * repeat):
            x()
        torch.cuda.synchronize()
        if x is not c2:
            del x
        torch.cuda.empty_cache()
    log("pmc pass done")
    return 0


# ------------------------------------------------------- counter summaries

def _kernel_tag(name: str):
    """The LEG_KERNELS entry a demangled kernel name is (None for other kernels)."""
    tags = {k for ks in LEG_KERNELS.values() for k in ks}
    for t in sorted(tags, key=len, reverse=True):
        if f"::{t}(" in name:
            return t
    return None


def _plan_slots() -> dict:
    """For every kernel, the leg of each of its dispatches in the pmc pass, in order."""
    slots: dict = {}
    for leg, n in PMC_PLAN:
        for _ in range(n):
            for k in LEG_KERNELS[leg]:
                slots.setdefault(k, []).append(leg)
    return slots


def _by_leg(per_dispatch: dict) -> dict:
    """{(dispatch id, kernel name): value} -> {leg: {kernel tag: [values]}} by dispatch order."""
    slots = _plan_slots()
    seen: dict = {}
    for (did, name) in sorted(per_dispatch, key=lambda x: int(x[0])):
        tag = _kernel_tag(name)
        if tag is None:
            continue
        seen.setdefault(tag, []).append(per_dispatch[(did, name)])
    out: dict = {}
    for tag, vals in seen.items():
        plan = slots.get(tag, [])
        # the pass may run the plan's calls `repeat` times over: each slot then stands for repeat dispatches
        if not plan or len(vals) % len(plan) != 0:
            raise SystemExit(f"{tag}: {len(vals)} dispatches, the plan has {len(plan)} (times a whole repeat)")
        rep = len(vals) // len(plan)
        for j, leg in enumerate(plan):
            out.setdefault(leg, {}).setdefault(tag, []).extend(vals[j * rep:(j + 1) * rep])
    return out


def _read_counters(d: str, counter: str) -> dict:
    """{(dispatch id, kernel name): value} of `counter` (summed over its
    instances) from a rocprofv3 --pmc run."""
    import csv

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    vals: dict = {}
    for f in files:
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") != counter:
                continue
            key = (row.get("Dispatch_Id"), row.get("Kernel_Name"))
            vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    return vals


def summarize_pmc(fetch_dir: str, write_dir: str) -> int:
    """HBM bytes per launch of each attention kernel, per workload, from two
    counter runs.  The counters are calibrated against the known-size device
    copy of the pass (it moves COPY_BYTES each way): factor = true bytes /
    counted bytes, applied to every kernel."""
    fetch = _read_counters(fetch_dir, "FETCH_SIZE")
    write = _read_counters(write_dir, "WRITE_SIZE")
    copy_f = [v for (i, n), v in fetch.items() if "copybuffer" in n.lower()]
    copy_w = [v for (i, n), v in write.items() if "copybuffer" in n.lower()]
    if not copy_f or not copy_w:
        raise SystemExit("copy kernel not found")
    f_factor = (COPY_BYTES / 1024.0) / max(copy_f)
    w_factor = (COPY_BYTES / 1024.0) / max(copy_w)
    fl, wl = _by_leg(fetch), _by_leg(write)
    out = {"source_sha256": source_digest(), "copy_bytes": COPY_BYTES, "fetch_factor": f_factor,
           "write_factor": w_factor, "plan": PMC_PLAN,
           "command": "rocprofv3 --pmc FETCH_SIZE -f csv -d <fetch dir> -o run -- python3 bench.py --pmc-pass ; "
                      "the same with --pmc WRITE_SIZE ; python3 bench.py --summarize-pmc <fetch dir> <write dir>",
           "legs": {}}
    for leg in fl:
        out["legs"][leg] = {}
        for tag, fv in fl[leg].items():
            wv = wl.get(leg, {}).get(tag, [0.0])
            out["legs"][leg][tag] = {"workload": LEG_WORKLOAD[leg], "dispatches": len(fv),
                                     "fetch_kib_raw": [round(x, 1) for x in fv], "write_kib_raw": [round(x, 1) for x in wv],
                                     "fetch_bytes": float(np.mean(fv)) * 1024 * f_factor,
                                     "write_bytes": float(np.mean(wv)) * 1024 * w_factor}
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out, indent=1))
    return 0


def summarize_counters(dirs: list) -> int:
    """Mean per dispatch of every counter found in the --pmc runs (one
    counter set per run), by workload and kernel, plus two derived ratios
    for the attention kernels: VALU instructions per MFMA instruction, and
    the fraction of MFMA-busy cycles in which VALU work issued beside it."""
    import csv

    names = set()
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                names.add(row["Counter_Name"])
    out = {"source_sha256": source_digest(), "plan": PMC_PLAN, "runs": len(dirs),
           "command": "rocprofv3 --pmc <up to 8 SQ counters> -f csv -d <dir> -o run -- python3 bench.py --pmc-pass "
                      "(one run per counter set) ; python3 bench.py --summarize-counters <dir> ...",
           "legs": {}}
    for name in sorted(names):
        vals: dict = {}
        for d in dirs:
            try:
                vals.update(_read_counters(d, name))
            except SystemExit:
                pass
        if not vals:
            continue
        for leg, per in _by_leg(vals).items():
            for tag, v in per.items():
                out["legs"].setdefault(leg, {}).setdefault(tag, {})[name] = float(np.mean(v))
    for leg, per in out["legs"].items():
        for tag, c in per.items():
            if c.get("SQ_INSTS_MFMA"):
                if "SQ_INSTS_VALU" in c:
                    c["valu_per_mfma"] = round(c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"], 3)
            if c.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in c:
                c["coexec_per_mfma_busy"] = round(c["SQ_VALU_MFMA_COEXEC_CYCLES"] / c["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
    path = os.path.join(ROOT, "profiles", "sq_counters.json")
    json.dump(out, open(path, "w"), indent=1)
    print(json.dumps(out, indent=1))
    return 0


def summarize_trace(d: str) -> int:
    """Kernel durations per workload from a `rocprofv3 --kernel-trace` run of
    `bench.py --pmc-pass --repeat R`: mean, median, min and max (us) of each
    kernel's dispatches in each leg, and the leg's algorithmic rate at the
    mean and the median."""
    import csv

    traces = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not traces:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    dur = {}
    for f in traces:
        for row in csv.DictReader(open(f)):
            dur[(row["Dispatch_Id"], row["Kernel_Name"])] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
    work = {leg: ("flop", prefill_flops(workloads.prefill_config(PREFILL_LEGS[leg]))) for leg in PREFILL_LEGS}
    work["c6"] = ("flop", chunked_flops(workloads.chunked_config(CHUNKED_CONFIG)))
    work["bwd_c2"] = ("flop", backward_flops(workloads.prefill_config(PREFILL_LEGS["c2"])))
    work["c5"] = ("byte", decode_bytes(workloads.decode_config(DECODE_CONFIG, with_values=False)))
    out = {"source_sha256": source_digest(), "plan": PMC_PLAN, "unit": "us",
           "command": "rocprofv3 --kernel-trace --stats -f csv -d <dir> -o run -- python3 bench.py --pmc-pass "
                      "--repeat R ; python3 bench.py --summarize-trace <dir>",
           "legs": {}}
    for leg, per in _by_leg(dur).items():
        entry = {"workload": LEG_WORKLOAD[leg], "kernels": {}}
        call_mean = call_median = 0.0
        for tag, vals in per.items():
            v = np.array(vals)
            entry["kernels"][tag] = {"dispatches": int(v.size), "mean": round(float(v.mean()), 2),
                                     "median": round(float(np.median(v)), 2), "min": round(float(v.min()), 2),
                                     "max": round(float(v.max()), 2)}
            call_mean += float(v.mean())
            call_median += float(np.median(v))
        kind, amount = work[leg]
        if kind == "flop":
            entry["tflops_at_mean"] = round(amount / (call_mean * 1e-6) / 1e12, 1)
            entry["tflops_at_median"] = round(amount / (call_median * 1e-6) / 1e12, 1)
        else:
            entry["gbs_at_mean"] = round(amount / (call_mean * 1e-6) / 1e9, 1)
            entry["gbs_at_median"] = round(amount / (call_median * 1e-6) / 1e9, 1)
        out["legs"][leg] = entry
    print(json.dumps(out, indent=1))
    return 0


def summarize_clock(d: str) -> int:
    """Cycles, shader clock and cycle-based MFMA utilisation per kernel and workload.

    GRBM_GUI_ACTIVE counts busy GPU cycles per die; per dispatch it is summed
    over the dies and divided by their number.  The kernel-trace duration of
    the same dispatch gives the clock it ran at.  MFMA utilisation in cycles
    = algorithmic flops / (cycles x whole-GPU dense bf16 flops per clock):
    the fraction of peak the kernel reaches at whatever clock the chip held.
    """
    import csv

    traces = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    counters = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not traces or not counters:
        raise SystemExit(f"need kernel_trace.csv and counter_collection.csv under {d}")
    dur, name = {}, {}
    for f in traces:
        for row in csv.DictReader(open(f)):
            dur[row["Dispatch_Id"]] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
            name[row["Dispatch_Id"]] = row["Kernel_Name"]
    cyc = {k: v for k, v in _read_counters(d, "GRBM_GUI_ACTIVE").items()}
    both = {(i, n): (v / NUM_XCD, dur[i]) for (i, n), v in cyc.items() if i in dur}
    flops = {leg: prefill_flops(workloads.prefill_config(PREFILL_LEGS[leg])) for leg in PREFILL_LEGS}
    flops["c6"] = chunked_flops(workloads.chunked_config(CHUNKED_CONFIG))
    out = {"source_sha256": source_digest(), "plan": PMC_PLAN,
           "command": "rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE -f csv -d <dir> -o run -- "
                      "python3 bench.py --pmc-pass ; python3 bench.py --summarize-clock <dir>",
           "legs": {}}
    for leg, per in _by_leg(both).items():
        out["legs"][leg] = {}
        for tag, vals in per.items():
            if tag == "decode_combine_kernel<128>":
                continue   # ~8 us: too short for the per-die busy counter to bracket reliably
            c = np.array([v[0] for v in vals])
            t = np.array([v[1] for v in vals], dtype=np.float64)
            k = {"workload": LEG_WORKLOAD[leg], "dispatches": len(vals), "cycles": [round(x) for x in c],
                 "ns": [int(x) for x in t], "sclk_ghz": [round(x, 3) for x in c / t]}
            if leg in flops and tag == LEG_KERNELS[leg][0]:
                k["mfma_util_cycles"] = [round(float(flops[leg] / (x * MFMA_FLOP_PER_CLK)), 4) for x in c]
            out["legs"][leg][tag] = k
    json.dump(out, open(CLOCK_FILE, "w"), indent=1)
    print(json.dumps(out, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
