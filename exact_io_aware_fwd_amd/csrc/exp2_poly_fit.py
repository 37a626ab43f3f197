"""Fit the coefficients of the software 2^f in exp2_poly.hpp.

2^x is computed as 2^n * p(f) with n = rint(x) and f = x - n in [-1/2, 1/2]
(Cody and Waite's range reduction).  p is the degree-4 polynomial that
minimises the largest relative error |p(f) / 2^f - 1| on that interval,
approximated by iteratively reweighted least squares (Lawson's algorithm):
each pass solves a weighted least-squares fit and multiplies the weights by
the current error, which drives the fit toward equal-ripple error.  The
coefficients are then rounded to float32, and the error is measured again
for the float32 Horner evaluation the kernel does.

    python exact_io_aware_fwd_amd/csrc/exp2_poly_fit.py
"""
import numpy as np

DEGREE = 4


def fit(degree: int = DEGREE, passes: int = 60):
    f = np.linspace(-0.5, 0.5, 20001)
    y = np.exp2(f)
    a = np.vander(f, degree + 1, increasing=True) / y[:, None]   # (p(f) - 2^f) / 2^f = a c - 1
    w = np.full(f.size, 1.0 / f.size)
    for _ in range(passes):
        sw = np.sqrt(w)
        c, *_ = np.linalg.lstsq(a * sw[:, None], sw, rcond=None)
        e = np.abs(a @ c - 1.0)
        w = w * e
        w /= w.sum()
    return c.astype(np.float32)


def horner_f32(c: np.ndarray, f: np.ndarray) -> np.ndarray:
    p = np.full(f.shape, c[-1], dtype=np.float32)
    for k in range(len(c) - 2, -1, -1):
        p = (p * f + c[k]).astype(np.float32)
    return p


def max_relative_error(c: np.ndarray) -> float:
    f = np.linspace(-0.5, 0.5, 200001).astype(np.float32)
    return float(np.abs(horner_f32(c, f).astype(np.float64) / np.exp2(f.astype(np.float64)) - 1.0).max())


if __name__ == "__main__":
    c = fit()
    for k, x in enumerate(c):
        print(f"constexpr float kExp2C{k} = {float(x):.9e}f;")
    print(f"// largest relative error in float32 Horner form: {max_relative_error(c):.3e}")
