"""Pins for the oracle's EWQ matrix entropy (softmax over the flattened matrix,
Shannon entropy in nats) and block entropy / tiers."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle
from tests import _brute

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_constant_matrix_is_log_n():
    # softmax of a constant matrix is uniform: H = ln n exactly
    for shape, c in [((4, 8), 0.0), ((256, 512), 0.37), ((3, 7), -2.5)]:
        n = shape[0] * shape[1]
        h = oracle.matrix_entropy(np.full(shape, c))
        assert abs(h - math.log(n)) <= 4e-16 * math.log(n)


def test_two_value_closed_form():
    # k entries equal to a, n - k zeros: Z = k e^a + n - k, H = ln Z - k a e^a / Z
    rng = np.random.default_rng(1)
    for n, k, a in [(32, 1, 3.0), (1000, 10, 0.5), (4096, 4095, -1.0), (64, 32, 2.0)]:
        w = np.zeros(n)
        w[rng.choice(n, k, replace=False)] = a
        z = k * math.exp(a) + n - k
        expect = math.log(z) - k * a * math.exp(a) / z
        assert oracle.matrix_entropy(w.reshape(-1, 8) if n % 8 == 0 else w) == pytest.approx(expect, rel=1e-14, abs=1e-14)


def test_worked_two_logits():
    # logits [0, ln 3] -> p = [1/4, 3/4] -> H = ln 4 - (3/4) ln 3
    h = oracle.matrix_entropy(np.array([[0.0, math.log(3.0)]]))
    assert h == pytest.approx(math.log(4.0) - 0.75 * math.log(3.0), rel=1e-15)


def test_shift_and_permutation_invariance():
    rng = np.random.default_rng(2)
    w = rng.normal(0, 0.05, size=(64, 96))
    h = oracle.matrix_entropy(w)
    assert oracle.matrix_entropy(w + 0.75) == pytest.approx(h, rel=1e-14)
    perm = rng.permutation(w.size)
    assert oracle.matrix_entropy(w.ravel()[perm].reshape(96, 64)) == pytest.approx(h, rel=1e-14)
    assert oracle.matrix_entropy(w.T) == pytest.approx(h, rel=1e-14)


def test_bounds_and_small_sigma_trend():
    rng = np.random.default_rng(3)
    n = 1 << 16
    for sigma in [0.005, 0.02, 0.08]:
        w = rng.normal(0, sigma, size=n)
        h = oracle.matrix_entropy(w)
        assert 0 <= h <= math.log(n)
        # H ~ ln n - Var(w)/2 for small weights (trend, not exact)
        assert (math.log(n) - h) == pytest.approx(np.var(w) / 2, rel=0.15)
    # a dominant entry drives H toward 0
    w = np.zeros(1000)
    w[0] = 50.0
    assert 0 <= oracle.matrix_entropy(w) < 1e-15 * 1e6


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_library_routines(seed):
    rng = np.random.default_rng(seed)
    w = rng.normal(0, 0.3, size=(37, 53))
    w.ravel()[rng.choice(w.size, 20, replace=False)] *= 10
    h = oracle.matrix_entropy(w)
    h_torch = torch.distributions.Categorical(
        logits=torch.from_numpy(w.ravel().copy())).entropy().item()
    h_scipy = scipy.stats.entropy(scipy.special.softmax(w.ravel()))
    assert h == pytest.approx(h_torch, rel=1e-13)
    assert h == pytest.approx(h_scipy, rel=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_4x8(seed):
    rng = np.random.default_rng(100 + seed)
    w = rng.normal(0, 1.0, size=(4, 8))
    h = oracle.matrix_entropy(w)
    hb = _brute.entropy_mp(w.ravel())
    assert abs(h - float(hb)) <= 1e-14 * float(hb)


def test_bf16_values_exact_in_fp64():
    w = (0.02 * torch.randn(64, 64, generator=torch.Generator().manual_seed(5))).to(torch.bfloat16)
    a = w.float().numpy()
    h = oracle.matrix_entropy(a)
    hb = _brute.entropy_mp(a.ravel().tolist(), dps=40)
    assert abs(h - float(hb)) < 1e-13


def test_nonfinite_gives_nan():
    w = np.zeros((2, 4))
    w[1, 2] = np.inf
    assert math.isnan(oracle.matrix_entropy(w))
    w[1, 2] = np.nan
    assert math.isnan(oracle.matrix_entropy(w))


def test_empty_rejected():
    with pytest.raises(ValueError):
        oracle.matrix_entropy(np.zeros((0, 4)))


def test_golden_block_entropy():
    g = json.load(open(os.path.join(GOLD, "ewq_tiers.json")))["block_entropy"]
    hb = oracle.block_entropy(g["h_mat"], g["sizes"], g["block_id"], g["n_blocks"])
    assert hb.tolist() == g["h_block"]
    with pytest.raises(ValueError):
        oracle.block_entropy([1.0], [1], [1], 2)  # block 0 empty


def _sigma(expr):
    return float(eval(expr, {"sqrt": math.sqrt}))


def test_golden_tiers():
    g = json.load(open(os.path.join(GOLD, "ewq_tiers.json")))
    for case in g["cases"]:
        mu, sigma, t, tiers = oracle.ewq_tiers(case["h"], case["x"])
        assert mu == pytest.approx(case["mu"], abs=1e-15)
        assert sigma == pytest.approx(_sigma(case["sigma"]), rel=1e-15, abs=1e-15)
        assert t == pytest.approx(case["mu"] - case["x"] * _sigma(case["sigma"]), abs=1e-14)
        assert tiers.tolist() == case["tiers"], case
        assert oracle.ewq_order(case["h"]).tolist() == case["order"], case


def test_tiers_boundaries_exact():
    # a block exactly at T is tier 1 (<=); a block exactly at mu is tier 3 (>=)
    h = np.array([0.0, 2.0, 1.0, 1.0])   # mu = 1, sigma = sqrt(0.5)
    mu, sigma, t, tiers = oracle.ewq_tiers(h)
    assert mu == 1.0 and tiers[2] == 3 and tiers[3] == 3
    h = np.array([0.0, 2.0])             # mu = 1, sigma = 1, T = 0 == h[0]
    assert oracle.ewq_tiers(h)[3].tolist() == [1, 3]
    # ddof=1 reading behind a flag moves sigma by sqrt(n/(n-1))
    h = np.arange(5.0)
    assert oracle.ewq_tiers(h, ddof=1)[1] == pytest.approx(math.sqrt(2.5))
