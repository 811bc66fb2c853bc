"""Group-wise quantisation to a non-uniform code book (oracle).  Test infrastructure only.

[SINQ] "Huawei giới thiệu SINQ…" (asiadaily.org), section "Tiết kiệm bộ nhớ,
tốc độ và chất lượng trong thử nghiệm": besides the integer grid, the method
also works with non-uniform quantisation.  The page names the option and no
grid, so the readings here are this implementation's (listed as N4 in the
design notes):

C1  A code book is 2^b ascending levels in [-1, 1] (b = 2, 3, 4); the
    default is the normal-quantile book: l_k = P((k + 1/2) / 2^b) /
    P((2^b - 1/2) / 2^b), P the standard normal quantile function (cells of
    equal probability under N(0, 1), symmetric, largest level 1), rounded to
    fp32.  Balancing leaves rows and columns with unit std, which is what the
    book is shaped for.
C2  Groups are g consecutive columns of a row of the balanced matrix
    x = (w * (1/s_i)) * (1/t_j) (the fp32 sequence of the integer quantiser);
    each group is scaled by its largest |x|, a (fp32, exact).
C3  The code of x is the level nearest to y = x * (1/a) (fp32), decided by
    the fp32 midpoints m_k = (l_k + l_{k+1}) * 0.5: code = #{k : y > m_k}, so
    a tie goes to the lower level.  a = 0 (or 1/a not finite) gives y = 0.
C4  Codes are packed b bits LSB-first per row like the integer codes;
    scales are fp32 [rows, cols / g]; there is no zero-point.
C5  Dequantisation: w' = ((a * l_code) * s_i) * t_j in fp32, each product
    rounded once.
"""
from __future__ import annotations

import numpy as np
from scipy.stats import norm

F32 = np.float32


def normal_levels(bits: int) -> np.ndarray:
    """The default normal-quantile code book (C1), fp32, ascending."""
    n = 1 << bits
    q = norm.ppf((np.arange(n, dtype=np.float64) + 0.5) / n)
    return (q / q[-1]).astype(F32)


def midpoints(levels) -> np.ndarray:
    lv = np.asarray(levels, dtype=F32)
    return ((lv[:-1] + lv[1:]).astype(F32) * F32(0.5)).astype(F32)


def quantize_codebook_f32(w, s, t, bits: int, group: int, levels):
    """(codes int [rows, cols], scales fp32 [rows, cols / group]) (C2, C3)."""
    a = np.asarray(w)
    rows, cols = a.shape
    x = a.astype(F32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        if s is not None:
            x = (x * (F32(1.0) / np.asarray(s, dtype=F32))[:, None]).astype(F32)
        if t is not None:
            x = (x * (F32(1.0) / np.asarray(t, dtype=F32))[None, :]).astype(F32)
    xg = x.reshape(rows, cols // group, group)
    amax = np.max(np.abs(xg), axis=2).astype(F32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        inv = (F32(1.0) / amax).astype(F32)
        ok = np.isfinite(inv)
        y = (xg * np.where(ok, inv, F32(0))[:, :, None]).astype(F32)
    m = midpoints(levels)
    codes = np.zeros(y.shape, dtype=np.int64)
    for mk in m:
        codes += (y > mk)
    return codes.reshape(rows, cols), amax


def dequantize_codebook_f32(codes, scales, s, t, group: int, levels) -> np.ndarray:
    """w' = ((a * l_code) * s_i) * t_j, fp32 (C5)."""
    q = np.asarray(codes)
    rows, cols = q.shape
    lv = np.asarray(levels, dtype=F32)
    a = np.repeat(np.asarray(scales, dtype=F32), group, axis=1)
    y = (a * lv[q]).astype(F32)
    if s is not None:
        y = (y * np.asarray(s, dtype=F32)[:, None]).astype(F32)
    if t is not None:
        y = (y * np.asarray(t, dtype=F32)[None, :]).astype(F32)
    return y
