"""Pins for the oracle's SINQ dual-axis Sinkhorn std balancing."""
import math
import statistics

import numpy as np
import pytest

import oracle
from tests import _brute
import woqdata


def _w(rows, cols, seed, sigma=0.02):
    return woqdata.random_matrix(rows, cols, seed, std=sigma).float().numpy().astype(np.float64)


def test_zero_iterations_is_identity():
    s, t = oracle.sinkhorn_std(_w(8, 16, 0), 0)
    assert np.all(s == 1) and np.all(t == 1)


def test_one_iteration_matches_statistics_pstdev():
    # after one (row, column) step from t = 1: s_i = pstdev(row i),
    # t_j = pstdev(column j of W / s)  -- via the stdlib's exact pstdev
    rng = np.random.default_rng(7)
    w = rng.normal(0.3, 0.05, size=(6, 9))  # rows with a large offset: centring matters
    s, t = oracle.sinkhorn_std(w, 1)
    s_ref = [statistics.pstdev(row.tolist()) for row in w]
    assert s == pytest.approx(s_ref, rel=1e-13)
    wd = w / np.array(s_ref)[:, None]
    t_ref = [statistics.pstdev(wd[:, j].tolist()) for j in range(w.shape[1])]
    assert t == pytest.approx(t_ref, rel=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_brute_force_4x8(seed):
    rng = np.random.default_rng(200 + seed)
    w = rng.normal(0, 1.0, size=(4, 8))
    for k in (1, 2, 5):
        s, t = oracle.sinkhorn_std(w, k)
        sb, tb = _brute.sinkhorn_mp(w.tolist(), k)
        assert s == pytest.approx(sb, rel=1e-12)
        assert t == pytest.approx(tb, rel=1e-12)


def test_convergence_invariant():
    # the fixed point: every column std of W/(s t^T) is 1 after a column step,
    # and the row stds become equal to one another (a common value r near 1)
    w = _w(256, 512, 1)
    for k, spread_bound in [(4, 1e-2), (8, 1e-4), (16, 1e-8), (24, 1e-12)]:
        s, t = oracle.sinkhorn_std(w, k)
        b = w / np.outer(s, t)
        col = b.std(axis=0)
        row = b.std(axis=1)
        assert np.max(np.abs(col - 1)) < 1e-12
        assert (row.max() - row.min()) / row.mean() < spread_bound
        assert abs(row.mean() - 1) < 5.0 / min(w.shape)


def test_spread_decays_geometrically():
    w = _w(128, 256, 2)
    spreads = []
    for k in (2, 4, 6, 8):
        s, t = oracle.sinkhorn_std(w, k)
        row = (w / np.outer(s, t)).std(axis=1)
        spreads.append((row.max() - row.min()) / row.mean())
    assert all(b < a * 0.5 for a, b in zip(spreads, spreads[1:])), spreads


def test_textbook_sinkhorn_knopp_reduction():
    # For W = [[A, -A], [-A, A]] every row and column has zero mean under any
    # scaling that keeps the two halves equal (and the iteration keeps them
    # equal), so the centred std is the RMS.  Then a_i = 1/s_i^2, b_j = 1/t_j^2
    # are exactly the Sinkhorn-Knopp factors of B = W o W with row sums = cols
    # and column sums = rows.
    rng = np.random.default_rng(9)
    a = rng.normal(0, 1, size=(3, 5))
    w = np.block([[a, -a], [-a, a]])
    rows, cols = w.shape
    for k in (1, 3, 8):
        s, t = oracle.sinkhorn_std(w, k)
        u, v = _brute.textbook_sinkhorn_knopp((w * w).tolist(), float(cols), float(rows), k)
        assert (1 / s ** 2) == pytest.approx(u, rel=1e-12)
        assert (1 / t ** 2) == pytest.approx(v, rel=1e-12)


def test_equivariances():
    w = _w(32, 48, 3)
    s, t = oracle.sinkhorn_std(w, 6)
    s2, t2 = oracle.sinkhorn_std(3.5 * w, 6)
    assert s2 == pytest.approx(3.5 * s, rel=1e-12) and t2 == pytest.approx(t, rel=1e-12)
    d = np.linspace(0.5, 2.0, 32)
    s3, t3 = oracle.sinkhorn_std(d[:, None] * w, 6)
    assert s3 == pytest.approx(d * s, rel=1e-12) and t3 == pytest.approx(t, rel=1e-12)


def test_zero_lines_get_scale_one():
    w = _w(16, 24, 4)
    w[3, :] = 0.0
    w[:, 5] = 0.0
    s, t = oracle.sinkhorn_std(w, 5)
    assert s[3] == 1.0 and t[5] == 1.0
    assert np.all(np.isfinite(s)) and np.all(np.isfinite(t))
    # zero entries still count in the other lines' statistics
    s1, _ = oracle.sinkhorn_std(w, 1)
    assert s1[0] == pytest.approx(statistics.pstdev(w[0].tolist()), rel=1e-13)


def test_constant_matrix_fixed_point():
    s, t = oracle.sinkhorn_std(np.full((5, 7), 0.25), 4)
    assert np.all(s == 1) and np.all(t == 1)
    # constant rows (bf16 values): zero std at the first row step
    w = _w(6, 10, 5)
    w[2, :] = 0.015625
    s, _ = oracle.sinkhorn_std(w, 1)
    assert s[2] == 1.0


def test_line_std_constant_lines_exactly_zero():
    # numpy's std of a constant line may be ~1e-17; the oracle makes it 0
    a = np.full((3, 1000), 0.1)
    assert np.all(oracle.line_std(a, 1) == 0)
    assert math.isclose(oracle.line_std(np.array([[1.0, 3.0]]), 1)[0], 1.0)


def test_rms_variant_is_sinkhorn_knopp_on_squares():
    """Uncentred variant: a_i = 1/s_i^2, b_j = 1/t_j^2 are the Sinkhorn-Knopp
    factors of B = W o W with row sums = cols and column sums = rows, for any
    W without zero lines (no structure needed, unlike the centred case)."""
    rng = np.random.default_rng(12)
    w = rng.normal(0.3, 1, size=(6, 9)) * rng.uniform(0.2, 3.0, size=(6, 1))
    rows, cols = w.shape
    for k in (1, 2, 5, 12):
        s, t = oracle.sinkhorn_std(w, k, rms=True)
        u, v = _brute.textbook_sinkhorn_knopp((w * w).tolist(), float(cols), float(rows), k)
        assert (1 / s ** 2) == pytest.approx(u, rel=1e-12)
        assert (1 / t ** 2) == pytest.approx(v, rel=1e-12)


def test_rms_variant_brute_force_and_zero_lines():
    # one iteration by plain Python sums, and a zero row / column -> scale 1
    w = np.array([[1.0, -2.0, 0.5], [0.0, 0.0, 0.0], [3.0, 1.0, -1.0]])
    s, t = oracle.sinkhorn_std(w, 1, rms=True)
    rs = [math.sqrt(sum(x * x for x in row) / 3) or 1.0 for row in w.tolist()]
    assert s == pytest.approx(rs, rel=1e-15)
    cs = [math.sqrt(sum((w[i][j] / rs[i]) ** 2 for i in range(3)) / 3) or 1.0 for j in range(3)]
    assert t == pytest.approx(cs, rel=1e-15)
    assert s[1] == 1.0
    # centred and uncentred agree on zero-mean lines, differ otherwise
    z = np.array([[1.0, -1.0], [2.0, -2.0]])
    assert np.allclose(oracle.sinkhorn_std(z, 1)[0], oracle.sinkhorn_std(z, 1, rms=True)[0])
    assert not np.allclose(oracle.sinkhorn_std(w + 1, 3)[0], oracle.sinkhorn_std(w + 1, 3, rms=True)[0])
