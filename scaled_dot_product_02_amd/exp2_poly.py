"""The polynomial behind the forward's optional exp2 split (ATTN_FLAG_FWD_EXP_SPLIT).

With the flag, one in four of the softmax exponentials of each lane on the forward's interior tiles is
computed on the VALU instead of the transcendental unit: Cody-Waite range reduction (W. J. Cody and
W. Waite, Software Manual for the Elementary Functions, 1980: split the argument into an integer and a
remainder, evaluate the remainder, scale by a power of two) specialised to base 2, so the reduction is
exact: n = rint(x), f = x - n in [-1/2, 1/2], 2^x = 2^n * 2^f, and 2^f is a degree-5 polynomial
fitted here. Nothing of a vendor math library is used; the coefficients below are this module's own
least-squares fit, and csrc/attn_device.h holds them as float32 literals (a CPU test checks the two
agree and the error bound holds).

Fit: minimise the relative error sum over 4001 Chebyshev points of [-1/2, 1/2] of
(p(f) - 2^f) / 2^f in float64, then round the coefficients to float32.
"""
import numpy as np

DEGREE = 5


def fit(degree=DEGREE, points=4001):
    k = np.arange(points)
    f = 0.5 * np.cos(np.pi * (k + 0.5) / points)  # Chebyshev points of [-1/2, 1/2]
    target = np.exp2(f)
    a = np.vander(f, degree + 1, increasing=True) / target[:, None]  # relative-error weights
    c, *_ = np.linalg.lstsq(a, np.ones_like(f), rcond=None)
    return [float(np.float32(x)) for x in c]  # c0 + c1 f + ... + c5 f^5


def eval_f32(x, coeffs):
    """The kernel's arithmetic in float32: clamp, n = rint(x), f = x - n, Horner with fused multiply-add
    (emulated by float64 products rounded once), ldexp."""
    x = np.maximum(np.asarray(x, dtype=np.float32), np.float32(-127.0))
    n = np.rint(x).astype(np.float32)
    f = (x - n).astype(np.float32)
    c = [np.float32(v) for v in coeffs]
    p = np.full_like(f, c[-1])
    for ci in reversed(c[:-1]):
        p = (p.astype(np.float64) * f.astype(np.float64) + np.float64(ci)).astype(np.float32)
    return np.ldexp(p, n.astype(np.int32)).astype(np.float32)


def max_rel_error(coeffs, lo=-30.0, hi=8.0, samples=2000001):
    x = np.linspace(lo, hi, samples).astype(np.float32)
    got = eval_f32(x, coeffs).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    return float(np.max(np.abs(got - ref) / ref))


if __name__ == "__main__":
    c = fit()
    print("coefficients (float32):", ", ".join(f"{v:.9e}f" for v in c))
    print("max relative error on [-30, 8]:", max_rel_error(c))
