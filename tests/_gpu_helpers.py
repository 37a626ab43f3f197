"""Helpers shared by the GPU parity tests (not a test module)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys
import time

import numpy as np
import torch

import oracle

BF16_TOL = dict(max_abs=1e-2, mean_abs=1e-3, lse=1e-3)
F32_TOL = dict(max_abs=1e-5, mean_abs=1e-5, lse=1e-3)
# Sharp attention (ALiBi slopes, large scales) gives outputs of a few units,
# where bf16 itself is coarse: the output's rounding costs up to 2^-9 |o| and
# the bf16 softmax weights of the P V product another 2^-9 relative, so the
# bound grows by 2^-8 |o_ref| on top of the absolute 1e-2.
# Beside it, the output is compared with the oracle's output rounded to bf16
# (bf16_max_abs): every element must be within 1e-2 of it, or else exactly
# one bf16 step away from it.  One step is the most two roundings of nearly
# the same number can differ by when the exact value sits near the midpoint
# between two bf16 values, and at |o| >= 2 one step (2^-6 and up) is more
# than 1e-2 however accurate the unrounded result is.
BF16_SHARP_TOL = dict(max_abs=1e-2, mean_abs=1e-3, lse=1e-3, rel=2.0 ** -8, bf16_max_abs=1e-2)


def bf16_step(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits; 2^-133 below 2^-126)."""
    _, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Host array from the generators -> device tensor of the kernel dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def oracle_prefill(case: dict, rows=None):
    dt = case["dtype"]
    return oracle.attention(oracle.to_f64(case["q"], dt), oracle.to_f64(case["k"], dt), oracle.to_f64(case["v"], dt), case["scale"],
                            case["mask"], case["window"], case["doc_offsets"], rows=rows)


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray, tol: dict,
            label: str = "") -> dict:
    """Element-wise check against the oracle; returns the error summary."""
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    empty = np.isneginf(lse_ref)
    # rows that see no key: exactly O = 0 and LSE = -inf
    if empty.any():
        assert np.all(o_gpu[empty] == 0.0), f"{label}: fully masked rows must be 0"
        assert np.all(np.isneginf(lse_gpu[empty])), f"{label}: fully masked rows must have LSE -inf"
    assert np.all(np.isfinite(lse_gpu[~empty])), f"{label}: non-finite LSE on a visible row"
    err = np.abs(o_gpu - o_ref)
    # max-abs is checked on err - rel |o_ref| (rel 0: plain max-abs); mean-abs on err itself
    bound_err = err - tol.get("rel", 0.0) * np.abs(o_ref)
    lerr = np.abs(lse_gpu[~empty] - lse_ref[~empty]) if (~empty).any() else np.zeros(1)
    summary = dict(max_abs=float(err.max()) if err.size else 0.0, mean_abs=float(err.mean()) if err.size else 0.0,
                   lse_max_abs=float(lerr.max()))
    if "bf16_max_abs" in tol:
        ref16 = oracle.round_to_bf16(o_ref)
        err16 = np.abs(o_gpu - ref16)
        summary["max_abs_vs_bf16_ref"] = float(err16.max()) if err16.size else 0.0
        beyond = err16 > tol["bf16_max_abs"]
        summary["beyond_1e-2_vs_bf16_ref"] = int(beyond.sum())
        # each such element must be exactly one bf16 step from the rounded oracle
        one_step = err16[beyond] == bf16_step(ref16[beyond])
        summary["beyond_not_one_step"] = int((~one_step).sum())
    say(f"[parity] {label}: {summary}")
    assert np.all(np.isfinite(o_gpu)), f"{label}: non-finite output"
    if tol.get("rel", 0.0) > 0.0:
        worst = float(bound_err.max()) if err.size else 0.0
        assert worst <= tol["max_abs"], f"{label}: max of |err| - {tol['rel']} |o| is {worst} > {tol['max_abs']}"
    else:
        assert summary["max_abs"] <= tol["max_abs"], f"{label}: max-abs {summary['max_abs']} > {tol['max_abs']}"
    if "bf16_max_abs" in tol:
        assert summary["beyond_not_one_step"] == 0, \
            f"{label}: {summary['beyond_not_one_step']} elements more than 1e-2 and more than one bf16 step " \
            f"from the bf16-rounded oracle"
    assert summary["mean_abs"] <= tol["mean_abs"], f"{label}: mean-abs {summary['mean_abs']} > {tol['mean_abs']}"
    assert summary["lse_max_abs"] <= tol["lse"], f"{label}: LSE max-abs {summary['lse_max_abs']} > {tol['lse']}"
    return summary


def doc_tensor(case):
    if case["doc_offsets"] is None:
        return None
    return torch.from_numpy(case["doc_offsets"].astype(np.int32)).cuda()


def workers() -> int:
    """Host threads for the oracle: the cores this process may run on (at most 16)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def parallel_map(fn, items, label: str = ""):
    """fn over items on a thread pool, in order, one BLAS thread per worker
    (numpy releases the GIL inside its kernels).  Prints progress at every
    quarter of the items."""
    from threadpoolctl import threadpool_limits

    items = list(items)
    out = [None] * len(items)
    t0 = time.perf_counter()
    marks = {max(1, (len(items) * q) // 4) for q in (1, 2, 3, 4)}
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(workers()) as ex:
        futs = {ex.submit(fn, it): n for n, it in enumerate(items)}
        for done, f in enumerate(cf.as_completed(futs), 1):
            out[futs[f]] = f.result()
            if done in marks:
                say(f"[oracle] {label}: {done}/{len(items)} tasks, {time.perf_counter() - t0:.1f} s")
    return out


def oracle_prefill_by_head(case: dict, label: str = ""):
    """Every row of every (batch, query head) from the oracle, one (batch,
    head) slice per task: heads are independent, and query head h reads KV
    head h // (Hq / Hkv)."""
    dt = case["dtype"]
    q, k, v = oracle.to_f64(case["q"], dt), oracle.to_f64(case["k"], dt), oracle.to_f64(case["v"], dt)
    B, Hq, Nq, d = q.shape
    g = Hq // k.shape[1]
    o = np.empty_like(q)
    lse = np.empty((B, Hq, Nq))

    def one(bh):
        b, h = bh
        ob, lb = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, h // g:h // g + 1], v[b:b + 1, h // g:h // g + 1],
                                  case["scale"], case["mask"], case["window"], case["doc_offsets"])
        o[b, h], lse[b, h] = ob[0, 0], lb[0, 0]

    parallel_map(one, [(b, h) for b in range(B) for h in range(Hq)], label)
    return o, lse


def oracle_document_by_parts(case: dict, label: str = ""):
    """Every row of a document-masked prefill through the per-document
    reduction: rows [a, b) of document [a, b) are causal attention over keys
    [a, b) alone (the document mask is causal inside each document; Nq = Nk)."""
    assert case["mask"] == "document" and case["Nq"] == case["Nk"]
    dt = case["dtype"]
    q, k, v = oracle.to_f64(case["q"], dt), oracle.to_f64(case["k"], dt), oracle.to_f64(case["v"], dt)
    B, Hq, Nq, d = q.shape
    g = Hq // k.shape[1]
    off = [int(x) for x in case["doc_offsets"]]
    assert off[0] == 0 and off[-1] == Nq, "documents must cover every row"
    o = np.empty_like(q)
    lse = np.empty((B, Hq, Nq))

    def one(task):
        b, h, a, e = task
        hk = h // g
        ob, lb = oracle.attention(q[b:b + 1, h:h + 1, a:e], k[b:b + 1, hk:hk + 1, a:e], v[b:b + 1, hk:hk + 1, a:e],
                                  case["scale"], "causal")
        o[b, h, a:e], lse[b, h, a:e] = ob[0, 0], lb[0, 0]

    # longest documents first, so the pool does not end on one long task
    tasks = sorted(((b, h, a, e) for b in range(B) for h in range(Hq) for a, e in zip(off[:-1], off[1:]) if e > a),
                   key=lambda t: t[2] - t[3])
    parallel_map(one, tasks, label)
    return o, lse
