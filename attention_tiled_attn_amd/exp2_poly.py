"""Minimax fit of 2^f on [0, 1] for the kernels' software exp2.

    python -m attention_tiled_attn_amd.exp2_poly     # prints the coefficients

FlashAttention-4 moves part of the softmax exponentials from the hardware
exponential unit to a polynomial evaluated on the multiply-add units (Neuron
FA4 explainer, "FlashAttention-4: Built for Blackwell", forward-pass fixes).
The pages give no polynomial; this one is fitted here.

Form: 2^x = 2^n * p(f) with n = floor(x), f = x - n in [0, 1), and
p(f) = 1 + f * (a1 + f * (a2 + f * a3)) (degree 3: the softmax weights, which
are rounded to bf16 anyway) or with a4 f^4 added (degree 4: soft-capping's
tanh, whose error the cap multiplies). Pinning p(0) = 1 makes integer
arguments exact, and with the argument clamped to -127 (so n = -127, f = 0)
adding n to the exponent field of p = 1.0 gives exactly +0: a masked score
(-inf) still contributes nothing.

Method: the Remez exchange algorithm for the best weighted uniform
approximation, here on the relative error r(f) = (p(f) - 2^f) / 2^f of the
constrained form p(f) = 1 + f * q(f). Each step solves for q's coefficients
and the levelled error E on (degree + 1) reference points, where the
error alternates in sign, then moves the references to the extrema of r on
a dense grid, until the extrema are level to 1e-12.

The coefficients the kernels use are these, rounded to float32, in
csrc/exp2_poly.h; tests/test_exp2_poly.py checks that header against this
fit and the float32 evaluation against fp64 2^x.
"""
from __future__ import annotations

import numpy as np


def _basis(f: np.ndarray, degree: int) -> np.ndarray:
    # p(f) - 1 = a1 f + a2 f^2 + ... + a_degree f^degree
    return np.stack([f ** (j + 1) for j in range(degree)], axis=-1)


def fit(degree: int = 3, iters: int = 60, grid: int = 200001):
    """(a1 .. a_degree) and the levelled relative error E of the minimax fit."""
    xs = np.linspace(0.0, 1.0, grid)
    target = np.exp2(xs)
    m = degree + 1   # reference points
    # initial references: Chebyshev extrema mapped to (0, 1]; f = 0 is exact
    k = np.arange(m)
    ref = 0.5 * (1.0 - np.cos(np.pi * (k + 1) / m))
    E = 0.0
    a = np.zeros(degree)
    for _ in range(iters):
        # p(x_i) - 2^x_i = (-1)^i E 2^x_i  ->  basis . a - (-1)^i 2^x_i E = 2^x_i - 1
        t = np.exp2(ref)
        A = np.concatenate([_basis(ref, degree), (-(-1.0) ** k * t)[:, None]], axis=1)
        sol = np.linalg.solve(A, t - 1.0)
        a, E = sol[:degree], sol[degree]
        r = (1.0 + _basis(xs, degree) @ a - target) / target
        # new references: the extremum of r in each run of constant sign
        sign = np.sign(r)
        sign[sign == 0] = 1
        cuts = np.flatnonzero(np.diff(sign) != 0) + 1
        runs = np.split(np.arange(xs.size), cuts)
        ext = [run[np.argmax(np.abs(r[run]))] for run in runs]
        ext = [i for i in ext if xs[i] > 0.0] if len(ext) > m else ext
        if len(ext) > m:   # keep the m largest consecutive alternating extrema
            vals = np.abs(r[ext])
            best = max(range(len(ext) - m + 1), key=lambda j: vals[j:j + m].min())
            ext = ext[best:best + m]
        new = xs[np.array(ext)]
        if len(new) == m and np.allclose(new, ref, atol=1e-12, rtol=0):
            break
        if len(new) == m:
            ref = new
    err = np.abs((1.0 + _basis(xs, degree) @ a - target) / target).max()
    return a, abs(E), err


def exp2_poly_f32(x, a) -> np.ndarray:
    """The kernels' evaluation in float32 steps (max, floor, subtract, one
    fused multiply-add per coefficient (Horner), exponent add), for tests.
    A fused step forms the product exactly in float64 and rounds the sum to
    float32 (within one float64 rounding of the single rounding of a true
    fused multiply-add)."""
    x = np.maximum(np.asarray(x, dtype=np.float32), np.float32(-127.0))
    n = np.floor(x).astype(np.float32)
    f = (x - n).astype(np.float32).astype(np.float64)
    c = [np.float64(np.float32(v)) for v in a]
    t = np.full(x.shape, c[-1], dtype=np.float64).astype(np.float32)
    for cj in reversed(c[:-1]):
        t = (t.astype(np.float64) * f + cj).astype(np.float32)
    p = (t.astype(np.float64) * f + 1.0).astype(np.float32)
    bits = p.view(np.int32) + (n.astype(np.int32) << 23)
    return bits.view(np.float32)


if __name__ == "__main__":
    for d in (3, 4):
        a, E, err = fit(d)
        print(f"degree {d}: a1..a{d} =", ", ".join(f"{c:.17g}" for c in a))
        print("  float32:", ", ".join(f"{float(np.float32(c))!r}" for c in a))
        print(f"  levelled relative error {E:.6e}, max on the grid {err:.6e}")
