"""The code bar against the plain fp64 definition: packed codes equal the
definition's except at near ties (|u - floor(u) - 1/2| < 1e-5 for the
element's ratio u, or for its group's zero-point ratio), where they may
differ by one, and such differences are at most 1e-5 of all elements (the
caller sums the counts over everything it checked)."""
from __future__ import annotations

import numpy as np

import oracle

BUDGET = 1e-5


def affine(w, s, t, bits, group, q_gpu):
    """GPU codes (unpacked, uint8 [rows, cols]) against the fp64 definition fed
    the given s and t.  Asserts the near-tie rule element by element; returns
    (mismatches, elements)."""
    q64 = oracle.quantize_groupwise_f64(w, s, t, bits, group)[0]
    diff = q_gpu != q64
    n = int(diff.sum())
    if n:
        tie = oracle.near_tie_mask(w, s, t, bits, group)
        assert np.all(~diff | tie), f"{int((diff & ~tie).sum())} codes differ away from a tie"
        assert int(np.max(np.abs(q_gpu.astype(np.int16) - q64.astype(np.int16)))) <= 1
    return n, int(diff.size)


def end_to_end(w, s_ref, t_ref, bits, group, q_gpu):
    """GPU codes against the definition fed the oracle's own s and t: the
    codes may move by one where the scales' rounding (within 2e-5) crosses a
    boundary.  Returns (mismatches, elements)."""
    q64 = oracle.quantize_groupwise_f64(w, s_ref, t_ref, bits, group)[0]
    diff = q_gpu != q64
    if diff.any():
        assert int(np.max(np.abs(q_gpu.astype(np.int16) - q64.astype(np.int16)))) <= 1
    return int(diff.sum()), int(diff.size)


def ternary(w, q_gpu):
    """GPU ternary codes q in {-1, 0, 1} (int8) against the fp64 definition
    (beta = mean |W| not rounded).  Returns (mismatches, elements)."""
    q64 = oracle.ternary_quantize_f64(w)[0]
    diff = q_gpu != q64
    n = int(diff.sum())
    if n:
        tie = oracle.ternary_near_tie_mask(w)
        assert np.all(~diff | tie), f"{int((diff & ~tie).sum())} ternary codes differ away from a tie"
        assert int(np.max(np.abs(q_gpu.astype(np.int16) - q64.astype(np.int16)))) <= 1
    return n, int(diff.size)


def within_budget(counts):
    """counts: iterable of (mismatches, elements)."""
    bad = sum(c[0] for c in counts)
    tot = sum(c[1] for c in counts)
    assert tot > 0
    assert bad <= BUDGET * tot, f"{bad} mismatches in {tot} codes"
    return bad, tot
