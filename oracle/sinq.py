"""SINQ dual-axis Sinkhorn-style std balancing (oracle, fp64).  Test infrastructure only.

[SINQ] "Định tỷ lệ trên hai trục": every weight matrix gets one scale vector
along its rows and one along its columns.  [SINQ] "Chuẩn hóa Sinkhorn Knopp":
an iteration in the manner of Sinkhorn-Knopp alternately rescales rows and
columns so that their standard deviations reach target values (the goal is
not a doubly stochastic matrix).

Readings where the page is silent: the target is 1 (each line is divided by
its measured std); std is the centred population std (1/n); the row step comes
first, starting from t = 1; ``iters`` counts full (row, column) iterations; a
line whose entries are all equal has std 0 and then gets scale 1.  The
balanced matrix is W / (s t^T).

Variant (``rms=True``): the uncentred root mean square sqrt(mean x^2) in place
of the std, for comparing the two readings in the quality report; a line of
zeros gets scale 1.
"""
from __future__ import annotations

import numpy as np


def line_std(a: np.ndarray, axis: int) -> np.ndarray:
    """Centred population std along ``axis``; exactly 0 for constant lines."""
    a = np.asarray(a, dtype=np.float64)
    m = a.mean(axis=axis, keepdims=True)
    sd = np.sqrt(np.mean((a - m) ** 2, axis=axis))
    const = a.max(axis=axis) == a.min(axis=axis)
    sd[const] = 0.0
    return sd


def line_rms(a: np.ndarray, axis: int) -> np.ndarray:
    """Uncentred root mean square along ``axis``."""
    a = np.asarray(a, dtype=np.float64)
    return np.sqrt(np.mean(a * a, axis=axis))


def sinkhorn_std(w, iters: int, rms: bool = False):
    """Return (s, t): row scales [rows] and column scales [cols] in fp64.

    For k = 1..iters:  s_i <- std_j(W_ij / t_j);  t_j <- std_i(W_ij / s_i),
    each zero std replaced by 1 (``rms``: root mean square instead of std).
    """
    if iters < 0:
        raise ValueError("iters must be >= 0")
    a = np.asarray(w, dtype=np.float64)
    rows, cols = a.shape
    f = line_rms if rms else line_std
    s = np.ones(rows)
    t = np.ones(cols)
    for _ in range(iters):
        s = f(a / t[None, :], axis=1)
        s[s == 0] = 1.0
        t = f(a / s[:, None], axis=0)
        t[t == 0] = 1.0
    return s, t
