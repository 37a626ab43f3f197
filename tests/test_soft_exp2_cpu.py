"""The software 2^x of the soft_exp2 forward option (exp2_poly.hpp), built for
the host from the same source and checked against 2^x in fp64.

What it has to meet: relative error at most 3e-6 wherever the result is a
normal float (x >= -125.5; the fitted polynomial's own bound is 2.7e-6, plus
float32 rounding of the reduction x - rint(x) and of the Horner steps), an
absolute error below 2^-149 plus that on the subnormal results of
[-126, -125.5), exactly 0 below -126 and at -inf (masked scores), exactly 1
at 0 up to the bound, and 2^n exactly reproduced up to the same bound at
every integer n (the reduction leaves f = 0 there, so p(0) = C0 alone)."""
import math
import os
import re
import shutil
import struct
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_io_aware_fwd_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

PROGRAM = r"""
#include "exp2_poly.hpp"
#include <cstdio>
#include <cstring>
#include <cstdint>
int main() {
    uint32_t bits;
    while (scanf("%x", &bits) == 1) {
        float x, y;
        memcpy(&x, &bits, 4);
        y = xattn::soft_exp2(x);
        memcpy(&bits, &y, 4);
        printf("%08x\n", bits);
    }
    return 0;
}
"""


def f32_bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).view(np.uint32)


@pytest.fixture(scope="module")
def soft_exp2(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    d = tmp_path_factory.mktemp("soft_exp2")
    src, exe = d / "e.cpp", d / "e"
    src.write_text(PROGRAM)
    subprocess.run([HIPCC, "-std=c++17", "-O2", "--cuda-host-only", "-x", "hip", "-I", CSRC, str(src), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)

    def run(x: np.ndarray) -> np.ndarray:
        x = np.asarray(x, dtype=np.float32)
        inp = "\n".join(f"{b:08x}" for b in f32_bits(x)) + "\n"
        out = subprocess.run([str(exe)], input=inp, check=True, capture_output=True, text=True, timeout=120).stdout
        return np.array([int(t, 16) for t in out.split()], dtype=np.uint32).view(np.float32)
    return run


def test_relative_error_on_the_reduced_interval(soft_exp2):
    # every float32 in [-1/2, 1/2] near a uniform grid, plus its ends
    x = np.concatenate([np.linspace(-0.5, 0.5, 100001, dtype=np.float32), np.float32([-0.5, 0.5, 0.0, -0.0])])
    y = soft_exp2(x).astype(np.float64)
    rel = np.abs(y / np.exp2(x.astype(np.float64)) - 1.0)
    assert rel.max() <= 3e-6, float(rel.max())


def test_relative_error_over_the_softmax_range(soft_exp2):
    # the softmax arguments s * scale * log2(e) - max lie in (-inf, 0]; the
    # positive side holds for the same reason, up to 2^127
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-125.5, 0.0, 100000), rng.uniform(0.0, 127.0, 5000),
                        np.arange(-125, 128, dtype=np.float64),             # integers: f = 0
                        np.arange(-125, 127, dtype=np.float64) + 0.5,       # ties of rint
                        np.arange(-125, 127, dtype=np.float64) - 0.5]).astype(np.float32)
    x = x[(x >= -125.5) & (x <= 127.0)]
    y = soft_exp2(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    assert np.all(np.isfinite(y)) and np.all(y > 0)
    rel = np.abs(y / ref - 1.0)
    assert rel.max() <= 3e-6, (float(rel.max()), float(x[rel.argmax()]))


def test_subnormal_results_and_underflow_to_zero(soft_exp2):
    x = np.linspace(-126.0, -125.5, 2001, dtype=np.float32)
    y = soft_exp2(x).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    assert np.all(np.abs(y - ref) <= 3e-6 * ref + 2.0 ** -149)
    below = np.float32([-126.0001, -126.5, -127.0, -127.5, -130.0, -1e4, -3.0e38, -np.inf])
    y = soft_exp2(below)
    assert np.all(y == 0.0) and not np.any(np.signbit(y))


def test_exact_points(soft_exp2):
    y = soft_exp2(np.float32([0.0, -1.0, 1.0, -10.0]))
    assert np.all(np.abs(y.astype(np.float64) / np.float64([1.0, 0.5, 2.0, 2.0 ** -10]) - 1.0) <= 3e-6)


def test_coefficients_are_the_fit_scripts():
    """The header's coefficients are what exp2_poly_fit.py prints (to float32
    rounding of a least-squares solve), and they meet the bound the header
    states when evaluated as the script evaluates them."""
    sys.path.insert(0, CSRC)
    keep, sys.dont_write_bytecode = sys.dont_write_bytecode, True   # no cache directory among the sources
    try:
        import exp2_poly_fit
    finally:
        sys.path.pop(0)
        sys.dont_write_bytecode = keep
    text = open(os.path.join(CSRC, "exp2_poly.hpp")).read()
    got = {int(k): float(v) for k, v in re.findall(r"kExp2C(\d)\s*=\s*([-+0-9.eE]+)f", text)}
    assert sorted(got) == [0, 1, 2, 3, 4]
    c = exp2_poly_fit.fit()
    for k in range(5):
        assert math.isclose(got[k], float(c[k]), rel_tol=1e-6), (k, got[k], float(c[k]))
    assert exp2_poly_fit.max_relative_error(np.float32([got[k] for k in range(5)])) <= 2.8e-6
