"""Independent brute-force references for tiny inputs (mpmath / exact fractions).

These share no code with ``oracle/``: they restate each definition in
high-precision or exact arithmetic, straight from the formula, with no
shifting, vectorisation or reformulation, so that they pin the oracle.
"""
from __future__ import annotations

from fractions import Fraction

import mpmath


def entropy_mp(values, dps: int = 50):
    """-sum p ln p with p_i = exp(w_i) / sum_j exp(w_j), at ``dps`` digits."""
    with mpmath.workdps(dps):
        ws = [mpmath.mpf(float(v)) for v in values]
        z = mpmath.fsum(mpmath.exp(w) for w in ws)
        h = mpmath.mpf(0)
        for w in ws:
            p = mpmath.exp(w) / z
            if p > 0:
                h -= p * mpmath.log(p)
        return h


def _pstd_mp(xs):
    n = len(xs)
    m = mpmath.fsum(xs) / n
    return mpmath.sqrt(mpmath.fsum((x - m) ** 2 for x in xs) / n)


def sinkhorn_mp(w, iters: int, dps: int = 50):
    """Alternating row / column centred population std, rows first from t = 1."""
    with mpmath.workdps(dps):
        a = [[mpmath.mpf(float(v)) for v in row] for row in w]
        rows, cols = len(a), len(a[0])
        s = [mpmath.mpf(1)] * rows
        t = [mpmath.mpf(1)] * cols
        for _ in range(iters):
            s = [_pstd_mp([a[i][j] / t[j] for j in range(cols)]) for i in range(rows)]
            s = [x if x != 0 else mpmath.mpf(1) for x in s]
            t = [_pstd_mp([a[i][j] / s[i] for i in range(rows)]) for j in range(cols)]
            t = [x if x != 0 else mpmath.mpf(1) for x in t]
        return [float(x) for x in s], [float(x) for x in t]


def rtn_argmin_codes(xs, delta, z, qmax):
    """For each x, the set of codes q in [0, qmax] minimising |x - (q - z) delta|.

    Exact rational arithmetic on the given floats.
    """
    d = Fraction(float(delta))
    out = []
    for x in xs:
        fx = Fraction(float(x))
        errs = [abs(fx - (q - int(z)) * d) for q in range(qmax + 1)]
        best = min(errs)
        out.append({q for q, e in enumerate(errs) if e == best})
    return out


def textbook_sinkhorn_knopp(b, row_target, col_target, iters: int):
    """Classic Sinkhorn-Knopp diagonal scaling u, v of a non-negative matrix b.

    Finds diag(u) b diag(v) with row sums ``row_target`` and column sums
    ``col_target``; v starts at 1 and u is updated first.
    """
    rows, cols = len(b), len(b[0])
    v = [1.0] * cols
    u = [1.0] * rows
    for _ in range(iters):
        u = [row_target / sum(b[i][j] * v[j] for j in range(cols)) for i in range(rows)]
        v = [col_target / sum(b[i][j] * u[i] for i in range(rows)) for j in range(cols)]
    return u, v
