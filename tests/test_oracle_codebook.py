"""Pins for the oracle's code-book (non-uniform grid) quantiser.

Each pin fixes the oracle against something other than itself: the normal
quantile at 50 digits (mpmath), the nearest level found by brute force in
exact arithmetic, the uniform symmetric book reduced to textbook rounding,
exact round trips of values that are levels, and the zero group.
"""
from fractions import Fraction

import mpmath
import numpy as np
import pytest

from oracle import codebook as cb
from oracle import rtn
import woqdata

F32 = np.float32


def _exact(x):
    """An mpf as an exact fraction."""
    sign, man, exp, _ = x._mpf_
    v = Fraction(int(man)) * (Fraction(2) ** int(exp))
    return -v if sign else v


def _mp_levels(bits):
    n = 1 << bits
    with mpmath.workdps(50):
        q = [mpmath.sqrt(2) * mpmath.erfinv(2 * (mpmath.mpf(k) + mpmath.mpf(1) / 2) / n - 1)
             for k in range(n)]
        return [q[k] / q[-1] for k in range(n)]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_normal_levels_against_the_quantile_at_50_digits(bits):
    lv = cb.normal_levels(bits)
    ref = _mp_levels(bits)
    assert lv.dtype == F32 and lv.shape == (1 << bits,)
    for a, b in zip(lv, ref):
        # the fp32 value is the rounding of the exact level: within half an ulp
        assert abs(Fraction(float(a)) - _exact(b)) <= Fraction(float(abs(np.spacing(a)))) / 2
    assert lv[-1] == 1.0 and lv[0] == -1.0
    assert np.array_equal(lv, -lv[::-1])            # symmetric
    assert np.all(np.diff(lv) > 0)


def test_two_bit_normal_book_closed_form():
    # n = 4: levels are the normal quantiles at 1/8, 3/8, 5/8, 7/8 over the one at 7/8
    lv = cb.normal_levels(2)
    with mpmath.workdps(30):
        r = mpmath.erfinv(mpmath.mpf(-1) / 4) / mpmath.erfinv(mpmath.mpf(3) / 4)
    assert lv[1] == F32(float(r))


def _brute_codes(y, levels):
    """Nearest level by exact distance, a tie to the lower level."""
    out = np.empty(y.shape, dtype=np.int64)
    L = [Fraction(float(v)) for v in levels]
    for i, v in enumerate(y.reshape(-1)):
        fv = Fraction(float(v))
        d = [abs(fv - lk) for lk in L]
        best = min(d)
        out.reshape(-1)[i] = d.index(best)
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codes_are_the_nearest_level(bits):
    """Away from the fp32 rounding of the midpoints, the midpoint count is the
    nearest level; at the rounded midpoints the fp32 rule decides (C3)."""
    rng = np.random.default_rng(40 + bits)
    lv = cb.normal_levels(bits)
    w = rng.standard_normal((6, 128)).astype(F32)
    q, a = cb.quantize_codebook_f32(w, None, None, bits, 32, lv)
    y = (w.reshape(6, 4, 32) * (F32(1) / a)[:, :, None]).astype(F32).reshape(6, 128)
    ref = _brute_codes(y, lv)
    m = cb.midpoints(lv)
    exact_mid = [(Fraction(float(lv[k])) + Fraction(float(lv[k + 1]))) / 2 for k in range(len(m))]
    for yi, qi, ri in zip(y.reshape(-1), q.reshape(-1), ref.reshape(-1)):
        if qi != ri:   # only possible between the exact and the rounded midpoint
            fy = Fraction(float(yi))
            assert any(min(Fraction(float(mk)), em) <= fy <= max(Fraction(float(mk)), em)
                       for mk, em in zip(m, exact_mid))
    assert np.mean(q == ref) > 0.999


def test_uniform_symmetric_book_is_textbook_rounding():
    """Levels -1 + 2k/(n-1) make the code book a uniform grid: the code is
    round((y + 1)(n - 1) / 2) with ties to the lower level."""
    n = 8
    lv = np.array([-1 + 2 * k / (n - 1) for k in range(n)], dtype=F32)
    rng = np.random.default_rng(5)
    w = rng.uniform(-3, 3, size=(4, 256)).astype(F32)
    q, a = cb.quantize_codebook_f32(w, None, None, 3, 64, lv)
    y = (w.reshape(4, 4, 64) / a[:, :, None].astype(np.float64)).reshape(4, 256)
    v = (y + 1) * (n - 1) / 2
    ref = np.ceil(v - 0.5).astype(np.int64)       # round half down
    ref = np.clip(ref, 0, n - 1)
    # midpoints are within fp32 rounding of the exact half-way points
    near = np.abs(v - np.round(v - 0.5) - 0.5) < 1e-5
    assert np.array_equal(q[~near], ref[~near])
    assert near.mean() < 1e-3


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_levels_round_trip_exactly(bits):
    """A group made of levels times a power of two holds its largest level
    (|l| = 1), so a is that power, y is the level itself, the code is its
    index and dequantisation returns the value exactly."""
    rng = np.random.default_rng(bits)
    lv = cb.normal_levels(bits)
    idx = rng.integers(0, 1 << bits, size=(5, 64))
    idx[:, ::16] = (1 << bits) - 1                  # every group holds level 1
    scale = F32(2.0) ** rng.integers(-8, 8, size=(5, 4)).astype(F32)
    w = (lv[idx] * np.repeat(scale, 16, axis=1)).astype(F32)
    q, a = cb.quantize_codebook_f32(w, None, None, bits, 16, lv)
    assert np.array_equal(a, scale)
    assert np.array_equal(q, idx)
    back = cb.dequantize_codebook_f32(q, a, None, None, 16, lv)
    assert np.array_equal(back, w)


def test_zero_group_and_sign_of_zero():
    lv = cb.normal_levels(4)
    w = np.zeros((2, 32), dtype=F32)
    w[1, :16] = 0.5
    q, a = cb.quantize_codebook_f32(w, None, None, 4, 16, lv)
    assert a.tolist() == [[0.0, 0.0], [0.5, 0.0]]
    # y = 0 is exactly the middle midpoint: the tie goes to the lower level
    assert np.all(q[0] == 7) and np.all(q[1, 16:] == 7)
    assert np.all(q[1, :16] == 15)
    back = cb.dequantize_codebook_f32(q, a, None, None, 16, lv)
    assert np.all(back[0] == 0) and np.all(back[1, :16] == 0.5)
    # -0.0 gives the same code as +0.0
    q2, _ = cb.quantize_codebook_f32(-w, None, None, 4, 16, lv)
    assert np.all(q2[0] == 7)


def test_balanced_values_match_the_integer_grid():
    """The code book sees the same balanced values as the integer grid: with
    8-bit affine codes of the same groups, x is recovered to within one step
    delta, so a = max |x| lies within delta of the affine reconstruction's
    largest magnitude."""
    w = woqdata.random_matrix(8, 128, 12, outlier_frac=0.02, outlier_mult=10.0).float().numpy()
    rng = np.random.default_rng(1)
    s = rng.uniform(0.5, 2, 8).astype(F32)
    t = rng.uniform(0.5, 2, 128).astype(F32)
    _, a = cb.quantize_codebook_f32(w, s, t, 4, 64, cb.normal_levels(4))
    q8, d8, z8 = rtn.quantize_groupwise_f32(w, s, t, 8, 64)
    x8 = rtn.dequantize_f32(q8, d8, z8, None, None, 64).reshape(8, 2, 64)
    amax8 = np.abs(x8).max(axis=2)
    assert np.all(np.abs(a - amax8) <= d8 * 0.5 * (1 + 1e-5))


def test_dequantize_product_order():
    """w' = ((a * l) * s) * t, each product rounded to fp32 once (C5)."""
    lv = cb.normal_levels(3)
    q = np.array([[0, 3, 5, 7]])
    a = np.array([[F32(0.7)]], dtype=F32)
    s = np.array([F32(1.3)], dtype=F32)
    t = np.array([1.1, 0.9, 2.0, 0.5], dtype=F32)
    out = cb.dequantize_codebook_f32(q, a, s, t, 4, lv)
    for j in range(4):
        v = F32(F32(F32(a[0, 0] * lv[q[0, j]]) * s[0]) * t[j])
        assert out[0, j] == v
