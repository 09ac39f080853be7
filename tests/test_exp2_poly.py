"""Pins of the cubic exp2 polynomial the forward can use on the FMA units.

The kernel's exp2_poly(x) clamps x to >= -127, splits x = n + f with
n = floor(x), evaluates p(f) = ((c3 f + c2) f + c1) f + c0 with fp32 FMAs and
returns ldexp(p, n).  For normal results the ldexp is exact, so the relative
error at x is the relative error of p at f = x - floor(x): sweeping every fp32
f in [2^-20, 1) exhaustively (and a dense sample below 2^-20, where p is
affine to working precision) covers every x in [-126, 8].  The bound to meet
is the bf16 half-ulp 2^-9 (the exponentials are rounded to bf16 next); the
minimax fit itself levels at about 7.5e-5.
"""
import os
import re

import numpy as np
import pytest

from exact_tiled_attention_27_amd import exp2_poly_fit

HEADER = os.path.join(os.path.dirname(exp2_poly_fit.__file__), "csrc", "fa_exp2_poly.hpp")


def header_coefficients():
    text = open(HEADER).read()
    vals = {}
    for m in re.finditer(r"kExp2Poly(\d) = ([0-9a-fx.p+-]+)f;", text):
        vals[int(m.group(1))] = float.fromhex(m.group(2))
    return np.array([vals[k] for k in range(4)], dtype=np.float64)


def fma32(a, b, c):
    """fp32 fused multiply-add: the product of two fp32 values is exact in
    float64, one rounding to fp32 at the end (a float64 intermediate rounding
    of the sum can shift the result by one fp32 ulp at most)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def poly32(f, c):
    c32 = c.astype(np.float32)
    p = fma32(np.full_like(f, c32[3]), f, np.full_like(f, c32[2]))
    p = fma32(p, f, np.full_like(f, c32[1]))
    return fma32(p, f, np.full_like(f, c32[0]))


def test_header_matches_the_fit():
    c = header_coefficients()
    fit = exp2_poly_fit.coefficients_f32().astype(np.float64)
    assert np.array_equal(c, fit)


def test_fit_equioscillates_at_the_minimax_level():
    c, E = exp2_poly_fit.remez_exp2()
    f = np.linspace(0.0, 1.0, 1_000_001)
    err = np.polynomial.polynomial.polyval(f, c) / 2.0 ** f - 1.0
    assert np.max(np.abs(err)) == pytest.approx(E, rel=1e-6)
    assert 5e-5 < E < 1e-4
    # equioscillation: exactly five runs of constant sign (degree + 2), each
    # reaching the levelled size, the ends included
    sign = np.sign(err)
    runs = np.split(np.abs(err), np.flatnonzero(np.diff(sign)) + 1)
    assert len(runs) == 5
    assert all(abs(r.max() - E) < 1e-8 for r in runs)
    assert abs(abs(err[0]) - E) < 1e-9 and abs(abs(err[-1]) - E) < 1e-9


def test_exhaustive_fraction_sweep_within_bf16_bound():
    c = header_coefficients()
    worst = 0.0
    # every fp32 in [2^-20, 1), one binade at a time
    for e in range(-20, 0):
        lo = np.float32(2.0 ** e).view(np.uint32)
        hi = np.float32(2.0 ** (e + 1)).view(np.uint32)
        f = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
        rel = np.abs(poly32(f, c).astype(np.float64) / np.exp2(f.astype(np.float64)) - 1.0)
        worst = max(worst, float(rel.max()))
    # below 2^-20: dense sample including 0 and the smallest normal
    f = np.concatenate([np.zeros(1, np.float32), np.geomspace(1.2e-38, 2.0 ** -20, 200_000).astype(np.float32)])
    rel = np.abs(poly32(f, c).astype(np.float64) / np.exp2(f.astype(np.float64)) - 1.0)
    worst = max(worst, float(rel.max()))
    _, E = exp2_poly_fit.remez_exp2()
    assert worst <= E + 4e-7          # the fit's level plus fp32 evaluation rounding
    assert worst < 2.0 ** -9          # far inside the bf16 bound


def test_split_and_clamp_cases():
    c = header_coefficients()

    def kernel_exp2(x):
        x = np.maximum(np.float32(x), np.float32(-127.0))
        n = np.floor(x)
        f = np.float32(x - n)
        return np.ldexp(poly32(np.array([f], np.float32), c)[0].astype(np.float64), int(n))

    for x in [0.0, 1.0, 8.0, -1.0, -0.3, -126.0, 7.999, 3.5, -17.25]:
        assert kernel_exp2(x) == pytest.approx(2.0 ** x, rel=8e-5)
    # -inf and anything below -127 clamp to 2^-127 (not 0): negligible
    assert kernel_exp2(-np.inf) == pytest.approx(2.0 ** -127, rel=8e-5)
    assert kernel_exp2(-1000.0) == pytest.approx(2.0 ** -127, rel=8e-5)
