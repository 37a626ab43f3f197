"""Helpers shared by the GPU parity tests (not a test module)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

BF16_TOL = dict(max_abs=1e-2, mean_abs=1e-3, lse=1e-3)
F32_TOL = dict(max_abs=1e-5, mean_abs=1e-5, lse=1e-3)
# Sharp attention (ALiBi slopes, large scales) gives outputs of a few units,
# where bf16 itself is coarse: the output's rounding costs up to 2^-9 |o| and
# the bf16 softmax weights of the P V product another 2^-9 relative, so the
# bound grows by 2^-8 |o_ref| on top of the absolute 1e-2.
BF16_SHARP_TOL = dict(max_abs=1e-2, mean_abs=1e-3, lse=1e-3, rel=2.0 ** -8)


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
    say(f"[parity] {label}: {summary}")
    assert np.all(np.isfinite(o_gpu)), f"{label}: non-finite output"
    if tol.get("rel", 0.0) > 0.0:
        worst = float(bound_err.max()) if err.size else 0.0
        assert worst <= tol["max_abs"], f"{label}: max of |err| - {tol['rel']} |o| is {worst} > {tol['max_abs']}"
    else:
        assert summary["max_abs"] <= tol["max_abs"], f"{label}: max-abs {summary['max_abs']} > {tol['max_abs']}"
    assert summary["mean_abs"] <= tol["mean_abs"], f"{label}: mean-abs {summary['mean_abs']} > {tol['mean_abs']}"
    assert summary["lse_max_abs"] <= tol["lse"], f"{label}: LSE max-abs {summary['lse_max_abs']} > {tol['lse']}"
    return summary


def doc_tensor(case):
    if case["doc_offsets"] is None:
        return None
    return torch.from_numpy(case["doc_offsets"].astype(np.int32)).cuda()
