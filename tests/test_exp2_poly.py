"""The kernels' software exp2 (csrc/exp2_poly.h): its coefficients are the
float32 rounding of the Remez fit in attention_tiled_attn_amd/exp2_poly.py,
the fit equioscillates (a minimax fit of the relative error), and the float32
evaluation stays within its error bound against fp64 2^x, with exact powers of
two at integers and exactly 0 for masked (-inf) scores."""
import os
import re

import numpy as np

from attention_tiled_attn_amd import exp2_poly

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "attention_tiled_attn_amd", "csrc", "exp2_poly.h")


import pytest

BOUNDS = {3: (8.0e-5, 8.6e-5), 4: (2.8e-6, 2.9e-6)}   # levelled error of each fit


def header_coeffs(degree):
    text = open(HEADER).read()
    name = "A" if degree == 3 else "B"
    return [np.float32(float(re.search(rf"kExp2{name}{i} = ([0-9.e+-]+)f;", text).group(1)))
            for i in range(1, degree + 1)]


@pytest.mark.parametrize("degree", [3, 4])
def test_header_matches_fit(degree):
    a, E, err = exp2_poly.fit(degree)
    lo, hi = BOUNDS[degree]
    assert lo < E < hi and abs(err - E) < 1e-9 * max(E, 1e-6)   # levelled: the error equioscillates
    assert header_coeffs(degree) == [np.float32(c) for c in a]
    assert abs(a[0] - np.log(2.0)) < 2e-3                        # slope of 2^f at 0


@pytest.mark.parametrize("degree", [3, 4])
def test_float32_evaluation_error_bound(degree):
    a = header_coeffs(degree)
    x = np.random.default_rng(0).uniform(-126.0, 8.0, 400_000).astype(np.float32)
    x = np.concatenate([x, np.linspace(-3, 3, 60001, dtype=np.float32)])
    got = exp2_poly.exp2_poly_f32(x, a).astype(np.float64)
    ref = np.exp2(x.astype(np.float64))
    rel = np.abs(got - ref) / ref
    # fit error plus a few float32 roundings of the evaluation
    assert rel.max() < BOUNDS[degree][1] + 6 * 2.0 ** -24, rel.max()


@pytest.mark.parametrize("degree", [3, 4])
def test_special_values(degree):
    a = header_coeffs(degree)
    ints = np.arange(-126, 9, dtype=np.float32)
    assert np.array_equal(exp2_poly.exp2_poly_f32(ints, a), np.exp2(ints))
    z = exp2_poly.exp2_poly_f32(np.array([-np.inf, -127.0, -1e30], dtype=np.float32), a)
    assert np.array_equal(z, np.zeros(3, dtype=np.float32)) and not np.signbit(z).any()
