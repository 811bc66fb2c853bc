"""EWQ's budgeted placement ([EWQ] "Giai ma EWQ & FastEWQ" (2kvn.com),
section "EWQ hoat dong nhu the nao?", step 3): the oracle against hand-worked
cases and properties of the rule, and the native host-side implementation
(ewq_budget_levels, C ABI) against the oracle.  No GPU is needed."""
import json
import os

import numpy as np
import pytest

import oracle
from weight_only_quantization_softmax_amd import _lib

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "ewq_budget.json")))


@pytest.mark.parametrize("case", GOLDEN["cases"], ids=[c["name"] for c in GOLDEN["cases"]])
def test_oracle_hand_cases(case):
    lev, total, fits = oracle.ewq_budget(case["h"], case["bytes"], case["level0"], case["budget"])
    assert lev.tolist() == case["levels"]
    assert total == case["total"] and fits == case["fits"]


def _random_case(rng, n=None, nl=4):
    n = n or int(rng.integers(1, 12))
    h = rng.normal(17.0, 0.01, n)
    if rng.random() < 0.3:   # entropy ties
        h[rng.integers(0, n, n // 2)] = h[0]
    base = rng.integers(100, 10_000, n)
    factors = np.array([0.16, 0.29, 0.51, 1.0])[:nl]
    lb = np.ceil(base[:, None] * factors[None, :] * rng.uniform(0.9, 1.1, (n, nl))).astype(np.int64)
    lb = np.sort(lb, axis=1)
    l0 = rng.integers(0, nl, n)
    lo, hi = lb[:, 0].sum(), lb[:, -1].sum()
    budget = int(rng.integers(max(lo - 200, 0), hi + 200))
    return h, lb, l0, budget


def test_oracle_properties():
    rng = np.random.default_rng(5)
    for _ in range(300):
        h, lb, l0, budget = _random_case(rng)
        lev, total, fits = oracle.ewq_budget(h, lb, l0, budget)
        assert total == sum(lb[b, lev[b]] for b in range(len(h)))
        start = sum(lb[b, l0[b]] for b in range(len(h)))
        if start <= budget:
            # promotion only, and maximal: no single further promotion fits
            assert fits and np.all(lev >= l0)
            for b in range(len(h)):
                if lev[b] + 1 < lb.shape[1]:
                    assert total - lb[b, lev[b]] + lb[b, lev[b] + 1] > budget
        else:
            # demotion only; stops as soon as it fits, or with every block at 0
            assert np.all(lev <= l0)
            assert fits or np.all(lev == 0)
            if fits:
                # the last step mattered: undoing any one demotion breaks the budget
                assert total <= budget


def test_native_matches_oracle():
    lib = _lib.load()
    import weight_only_quantization_softmax_amd as woq
    rng = np.random.default_rng(6)
    for _ in range(400):
        h, lb, l0, budget = _random_case(rng)
        ref = oracle.ewq_budget(h, lb, l0, budget)
        got = woq.ewq_budget_levels(h.tolist(), lb.tolist(), l0.tolist(), budget)
        assert got[0] == ref[0].tolist() and got[1] == ref[1] and got[2] == ref[2]
    assert lib is not None


def test_native_errors():
    import ctypes
    lib = _lib.load()
    h = (ctypes.c_double * 2)(1.0, 2.0)
    lb = (ctypes.c_int64 * 4)(1, 2, 1, 2)
    l0 = (ctypes.c_int32 * 2)(0, 1)
    out = (ctypes.c_int32 * 2)()
    tot = ctypes.c_int64()
    fits = ctypes.c_int32()
    call = lib.ewq_budget_levels
    assert call(h, lb, 2, 2, l0, 10, out, ctypes.byref(tot), ctypes.byref(fits)) == 0
    assert call(None, lb, 2, 2, l0, 10, out, ctypes.byref(tot), ctypes.byref(fits)) == 1
    assert call(h, lb, 0, 2, l0, 10, out, ctypes.byref(tot), ctypes.byref(fits)) == 10
    assert call(h, lb, 2, 0, l0, 10, out, ctypes.byref(tot), ctypes.byref(fits)) == 10
    assert call(h, lb, 2, 2, l0, -1, out, ctypes.byref(tot), ctypes.byref(fits)) == 2
    bad = (ctypes.c_int32 * 2)(0, 2)
    assert call(h, lb, 2, 2, bad, 10, out, ctypes.byref(tot), ctypes.byref(fits)) == 2
    nan = (ctypes.c_double * 2)(1.0, float("nan"))
    assert call(nan, lb, 2, 2, l0, 10, out, ctypes.byref(tot), ctypes.byref(fits)) == 11
