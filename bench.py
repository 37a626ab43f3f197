#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one causal bf16 prefill (B=4, Hq=Hkv=16, N=2048, d=128, the
headline workload) followed by one paged decode (64 sequences, Hq=32, Hkv=8,
d=128, context lengths uniform in [1024, 32768], 16-token pages, seeded
random page placement).  Inputs are seeded synthetic data, generated on the
host, copied once and resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Prints ONE JSON line.  `value` is the prefill's algorithmic TFLOP/s
(4·d·B·Hq·visible pairs per call ÷ the kernel's mean duration from HIP events
on the launch stream); the decode's algorithmic HBM GB/s is reported beside
it.  `cpu_baseline` is the fp64 numpy oracle timed on this host over a bounded
sample of the same prefill workload.

    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR

turns two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
`bench.py --pmc-pass` into profiles/hbm_traffic.json.

    python bench.py --summarize-clock DIR

turns one `rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE` run of
`bench.py --pmc-pass` into per-kernel GPU cycles, the shader clock the
kernel actually ran at (cycles / duration) and, for the prefill, the MFMA
utilisation in cycles (prefill C2, decode C5, chunked prefill C6):
profiles/sclk_prefill_c2_decode_c5.json.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
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
# every kernel the counter and clock summaries cover, with the workload it runs in bench.py
KERNEL_WORKLOADS = {
    "prefill_bf16_kernel<128, false>": PREFILL_CONFIG,
    "decode_split_kernel<128, false>": DECODE_CONFIG,
    "decode_combine_kernel<128>": DECODE_CONFIG,
    "paged_prefill_swz_kernel<false>": CHUNKED_CONFIG,
    "bwd_prep_kernel": "backward of " + PREFILL_CONFIG,
    "bwd_dq_kernel": "backward of " + PREFILL_CONFIG,
    "bwd_dkdv_kernel": "backward of " + PREFILL_CONFIG,
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CLOCK_FILE = os.path.join(ROOT, "profiles", "sclk_prefill_c2_decode_c5.json")
NUM_XCD = 8                   # GRBM_GUI_ACTIVE is counted once per accelerator die
MFMA_FLOP_PER_CLK = 256 * 4096  # dense bf16 MFMA, whole GPU, per shader clock
CSRC = os.path.join(ROOT, "exact_io_aware_fwd_amd", "csrc")
COPY_BYTES = 1 << 30          # known-size copy used to calibrate the HBM byte counters


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
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()


def measured_traffic(kernel_key: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none for this workload or the kernel sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    t = json.load(open(TRAFFIC_FILE))
    if t.get("source_sha256") != source_digest():
        return None
    k = t.get("kernels", {}).get(kernel_key)
    if not k or k.get("workload") != workload:
        return None
    return int(k["fetch_bytes"] + k["write_bytes"])


# -------------------------------------------------------------- CPU baseline

def cpu_baseline(c: dict, budget_s: float) -> dict:
    """The fp64 oracle, as it is, on whole (batch, head) slices of the prefill
    workload until the time budget is spent; TFLOP/s of algorithmic work."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        cores = max([int(x.get("num_threads", 1)) for x in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    per_head = 4 * c["d"] * visible_pairs(c["Nq"], c["Nk"], c["mask"], c["window"], c["doc_offsets"])
    g = c["Hq"] // c["Hkv"]
    heads = [(b, h) for b in range(c["B"]) for h in range(c["Hq"])]
    done = 0
    t0 = time.perf_counter()
    for b, h in heads:
        hk = h // g
        q = oracle.to_f64(c["q"][b:b + 1, h:h + 1], c["dtype"])
        k = oracle.to_f64(c["k"][b:b + 1, hk:hk + 1], c["dtype"])
        v = oracle.to_f64(c["v"][b:b + 1, hk:hk + 1], c["dtype"])
        oracle.attention(q, k, v, c["scale"], c["mask"], c["window"], c["doc_offsets"])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(done * per_head / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{PREFILL_CONFIG}: {done} of {len(heads)} (batch, head) slices, all {c['Nq']} rows each, "
                      f"{el:.1f} s fp64 numpy"}


# ------------------------------------------------------------------- GPU run

def to_dev(x: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill-config", default=PREFILL_CONFIG)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chunked", action="store_true", help="skip the chunked-prefill measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="short run for counter collection: a few steps plus one known-size copy")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-clock", metavar="DIR")
    args = ap.parse_args()

    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc)
    if args.summarize_clock:
        return summarize_clock(args.summarize_clock)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; multi-GPU runs are not part of "
                                   "this build (--gpus must be 1)"}))
        return 2

    import torch
    from exact_io_aware_fwd_amd import attn_fwd, attn_paged_decode, attn_paged_decode_workspace_size

    torch.cuda.set_device(0)
    log(f"generating inputs ({args.prefill_config}, {DECODE_CONFIG})")
    pc = workloads.prefill_config(args.prefill_config)
    dc = workloads.decode_config(DECODE_CONFIG)
    q, k, v = to_dev(pc["q"]), to_dev(pc["k"]), to_dev(pc["v"])
    doc = torch.from_numpy(pc["doc_offsets"]).cuda() if pc["doc_offsets"] is not None else None
    o = torch.empty_like(q)
    lse = torch.empty((pc["B"], pc["Hq"], pc["Nq"]), dtype=torch.float32, device="cuda")
    dq, dk, dv = to_dev(dc["q"]), to_dev(dc["k_pages"]), to_dev(dc["v_pages"])
    bt = torch.from_numpy(dc["block_table"]).cuda()
    sl = torch.from_numpy(dc["seq_lens"]).cuda()
    do = torch.empty_like(dq)
    dl = torch.empty((dc["num_seqs"], dc["Hq"]), dtype=torch.float32, device="cuda")
    ws = torch.empty(attn_paged_decode_workspace_size(dc["num_seqs"], dc["Hq"], dc["d"], dc["max_seq_len"]),
                     dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log("inputs resident on the GPU")

    def prefill():
        attn_fwd(q, k, v, scale=pc["scale"], mask=pc["mask"], window=pc["window"], doc_offsets=doc, out=o, lse=lse)

    def decode():
        attn_paged_decode(dq, dk, dv, bt, sl, max_seq_len=dc["max_seq_len"], scale=dc["scale"], workspace=ws,
                          out=do, lse=dl)

    if args.pmc_pass:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").normal_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        for _ in range(3):
            prefill()
            decode()
        torch.cuda.synchronize()
        if not args.no_chunked:
            time_chunked(3, 0)
        if not args.no_backward:
            time_backward(pc, q, k, v, o, lse, doc, 3, 0)
        log("pmc pass done")
        return 0

    K, W = args.steps, args.warmup
    for _ in range(W):
        prefill()
        decode()
    torch.cuda.synchronize()
    log(f"warmup done ({W} steps)")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(K):
        evs[i][0].record()
        prefill()
        evs[i][1].record()
        decode()
        evs[i][2].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = start.elapsed_time(end) / K
    pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    pre_mean, dec_mean = float(np.mean(pre_ms)), float(np.mean(dec_ms))
    log(f"timed {K} steps: {step_ms:.3f} ms/step (wall {wall:.2f} s); prefill {pre_mean*1e3:.1f} us, "
        f"decode {dec_mean*1e3:.1f} us")

    flops = prefill_flops(pc)
    tflops = flops / (pre_mean * 1e-3) / 1e12
    dbytes = decode_bytes(dc)
    gbs = dbytes / (dec_mean * 1e-3) / 1e9
    pkey = f"prefill_bf16_kernel<{pc['d']}, false>"
    ptraffic = measured_traffic(pkey, args.prefill_config)
    dtraffic = measured_traffic("decode_split_kernel<128, false>", DECODE_CONFIG)

    result = {
        "metric": "attn fwd TFLOP/s (% bf16 MFMA peak) causal prefill; paged decode HBM GB/s",
        "value": round(tflops, 2),
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
            "workload": f"{args.prefill_config} (B{pc['B']} Hq{pc['Hq']} Hkv{pc['Hkv']} N{pc['Nq']} d{pc['d']} "
                        f"{pc['mask']}) + {DECODE_CONFIG} (64 seqs, Hq32 Hkv8 d128, 16-token pages, "
                        f"{int(dc['seq_lens'].sum())} cached tokens)",
            "prefill_flop_per_call": flops,
            "prefill_us": round(pre_mean * 1e3, 2),
            "decode_bytes_per_call": dbytes,
            "decode_us": round(dec_mean * 1e3, 2),
            "parallelism": "single GPU",
        },
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": ptraffic,
            "kernel": pkey, "algorithmic_bytes": prefill_bytes(pc),
        },
        "decode": {
            "value": round(gbs, 1), "unit": "GB/s", "pct_of_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": dtraffic,
                         "kernel": "decode_split_kernel<128, false> + decode_combine_kernel<128> (one call)"},
        },
    }
    if not args.no_chunked:
        result["chunked_prefill"] = time_chunked(K, W)
    if not args.no_backward:
        result["backward"] = time_backward(pc, q, k, v, o, lse, doc, K, W)
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on host cores")
        result["cpu_baseline"] = cpu_baseline(pc, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


def backward_flops(c: dict) -> int:
    """The backward's five products per visible pair (recomputed scores, dP,
    dV, dK, dQ), 2 d flops each."""
    return 10 * c["d"] * c["B"] * c["Hq"] * visible_pairs(c["Nq"], c["Nk"], c["mask"], c["window"], c["doc_offsets"])


def time_backward(pc: dict, q, k, v, o, lse, doc, K: int, W: int) -> dict:
    """Backward of the headline prefill from its own o and lse (timed alone,
    after the step loop): algorithmic TFLOP/s against the bf16 MFMA peak."""
    import torch
    from exact_io_aware_fwd_amd import attn_bwd, attn_bwd_workspace_size

    do = to_dev(workloads.gen._draw(0, 5, (pc["B"], pc["Hq"], pc["Nq"], pc["d"]), "bf16"))
    ws = torch.empty(attn_bwd_workspace_size(pc["B"], pc["Hq"], pc["Nq"]), dtype=torch.uint8, device="cuda")
    kw = dict(scale=pc["scale"], mask=pc["mask"], window=pc["window"], doc_offsets=doc, workspace=ws)

    for _ in range(W):
        attn_bwd(q, k, v, o, do, lse, **kw)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        attn_bwd(q, k, v, o, do, lse, **kw)
        ev[i][1].record()
    torch.cuda.synchronize()
    us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    flops = backward_flops(pc)
    tf = flops / (us * 1e-6) / 1e12
    log(f"backward: {us:.1f} us, {tf:.1f} TFLOP/s")
    return {"value": round(tf, 2), "unit": "TFLOP/s", "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "us": round(us, 2), "flop_per_call": flops, "workload": f"backward of {PREFILL_CONFIG}",
            "kernels": "bwd_prep_kernel + bwd_dq_kernel + bwd_dkdv_kernel (one call)"}


def time_chunked(K: int, W: int) -> dict:
    """Chunked prefill over the paged cache (its own workload, timed alone
    after the step loop): algorithmic TFLOP/s against the bf16 MFMA peak."""
    import torch
    from exact_io_aware_fwd_amd import attn_paged_prefill

    c = workloads.chunked_config(CHUNKED_CONFIG)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    q, kp, vp = to_dev(c["q"]), to_dev(c["k_pages"]), to_dev(c["v_pages"])
    bt, sl, qo = i32(c["block_table"]), i32(c["seq_lens"]), i32(c["q_offsets"])
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")

    def call():
        attn_paged_prefill(q, kp, vp, bt, sl, qo, max_seq_len=c["max_seq_len"], max_q_len=c["max_q_len"],
                           scale=c["scale"], mask=c["mask"], out=o, lse=lse)

    for _ in range(W):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        call()
        ev[i][1].record()
    torch.cuda.synchronize()
    us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    flops = chunked_flops(c)
    tf = flops / (us * 1e-6) / 1e12
    log(f"chunked prefill: {us:.1f} us, {tf:.1f} TFLOP/s")
    return {"value": round(tf, 2), "unit": "TFLOP/s", "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "us": round(us, 2), "flop_per_call": flops,
            "workload": f"{CHUNKED_CONFIG} ({c['num_seqs']} seqs, Hq{c['Hq']} Hkv{c['Hkv']} d{c['d']}, "
                        f"{int(c['q_offsets'][-1])} chunk tokens over {int(c['seq_lens'].sum())} cached, causal)",
            "kernel": "paged_prefill_swz_kernel<false>" if c["d"] == 128 else f"paged_prefill_bf16_kernel<{c['d']}, false>"}


# ------------------------------------------------------- counter summaries

def _read_counters(d: str, counter: str) -> dict:
    """Per-dispatch values of `counter` (KiB), by kernel name, from a rocprofv3 --pmc run."""
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
    per_kernel: dict = {}
    for (_, name), v in vals.items():
        per_kernel.setdefault(name, []).append(v)
    return per_kernel


def summarize_pmc(fetch_dir: str, write_dir: str) -> int:
    """HBM bytes per launch of each attention kernel from two counter runs.

    The byte counters are calibrated against the known-size device copy of
    the --pmc-pass run (its largest copy dispatch moves COPY_BYTES each way):
    factor = true bytes / counted bytes, applied to every kernel.
    """
    fetch = _read_counters(fetch_dir, "FETCH_SIZE")
    write = _read_counters(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "copybuffer" in k.lower()]
    if not copy:
        raise SystemExit("copy kernel not found in the FETCH_SIZE run")
    ck = copy[0]
    f_factor = (COPY_BYTES / 1024.0) / max(fetch[ck])
    w_factor = (COPY_BYTES / 1024.0) / max(write[ck])
    out = {"source_sha256": source_digest(), "copy_kernel": ck, "copy_bytes": COPY_BYTES,
           "fetch_factor": f_factor, "write_factor": w_factor,
           "command": "rocprofv3 --pmc FETCH_SIZE -f csv -d <dir> -o run -- python3 bench.py --pmc-pass ; "
                      "the same with --pmc WRITE_SIZE ; python3 bench.py --summarize-pmc <fetch dir> <write dir>",
           "kernels": {}}
    for name in fetch:
        short = None
        for tag in KERNEL_WORKLOADS:
            if f"::{tag}" in name and (short is None or len(tag) > len(short)):
                short = tag
        if short is None:
            continue
        wl = KERNEL_WORKLOADS[short]
        fk = float(np.mean(fetch[name]))
        wk = float(np.mean(write.get(name, [0.0])))
        out["kernels"][short] = {"workload": wl, "dispatches": len(fetch[name]), "fetch_kib_raw": fk,
                                 "write_kib_raw": wk, "fetch_bytes": fk * 1024 * f_factor,
                                 "write_bytes": wk * 1024 * w_factor}
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out, indent=1))
    return 0


def summarize_clock(d: str) -> int:
    """Cycles, shader clock and cycle-based MFMA utilisation per attention kernel.

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
    cyc: dict = {}
    for f in counters:
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") == "GRBM_GUI_ACTIVE":
                cyc[row["Dispatch_Id"]] = cyc.get(row["Dispatch_Id"], 0.0) + float(row["Counter_Value"])
    flops = {"prefill_bf16_kernel<128, false>": prefill_flops(workloads.prefill_config(PREFILL_CONFIG)),
             "paged_prefill_swz_kernel<false>": chunked_flops(workloads.chunked_config(CHUNKED_CONFIG))}
    out = {"source_sha256": source_digest(),
           "command": "rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE -f csv -d <dir> -o run -- "
                      "python3 bench.py --pmc-pass ; python3 bench.py --summarize-clock <dir>",
           "kernels": {}}
    for tag, wl in KERNEL_WORKLOADS.items():
        if tag == "decode_combine_kernel<128>":
            continue   # ~14 us: too short for the per-die busy counter to bracket reliably
        # kernel names are demangled signatures: match the name, not a prefix of another
        ids = [i for i in dur if f"::{tag}(" in name[i] and i in cyc]
        if not ids:
            continue
        c = np.array([cyc[i] / NUM_XCD for i in ids])
        t = np.array([dur[i] for i in ids], dtype=np.float64)
        k = {"workload": wl, "dispatches": len(ids), "cycles_median": float(np.median(c)),
             "ns_median": float(np.median(t)), "sclk_ghz_median": float(np.median(c / t))}
        if tag in flops:
            k["mfma_util_cycles"] = float(flops[tag] / (np.median(c) * MFMA_FLOP_PER_CLK))
        out["kernels"][tag] = k
    json.dump(out, open(CLOCK_FILE, "w"), indent=1)
    print(json.dumps(out, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
