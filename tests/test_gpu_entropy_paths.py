"""The three ways a bf16 weight is counted by the entropy pass, each against
the oracle (entropy within 1e-12 relative, exponent histogram exact).

A weight whose magnitude lies in [2^-25, 2^6) lands in the window histogram;
zeros and NaN / inf are counted; any other value (tiny, subnormal, or
|w| >= 64) is kept as its bit pattern in a per-matrix list, summed in
sorted order.  When a work unit meets more such values than its LDS list
holds, or a matrix more than its list holds, the matrix is marked spilled
and its other values are recounted from the weights.  Every case below is
built to take one of these routes, on contiguous matrices and strided
views, and each result must not depend on the route or on scheduling.
"""
import numpy as np
import pytest
import torch

import woqdata
import weight_only_quantization_softmax_amd as woq
from oracle import df11, matrix_entropy

pytestmark = pytest.mark.gpu
DEV = "cuda"
UNIT = 1 << 19          # elements per work unit, at most
LDS_LIST = 240          # other values one work unit keeps
LIST_CAP = 8192         # other values one matrix keeps


def _base(rows, cols, seed, std=0.02):
    return woqdata.random_matrix(rows, cols, seed, std=std).float().numpy()


def _plant(w, n, seed, lo, hi):
    """Sets n distinct positions of w (numpy fp32) to +-values with
    magnitudes log-uniform in [lo, hi); returns w."""
    rng = np.random.default_rng(seed)
    flat = w.reshape(-1)
    pos = rng.choice(flat.size, size=n, replace=False)
    mag = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n))
    flat[pos] = np.where(rng.random(n) < 0.5, -mag, mag)
    return w


def _bf(w):
    return torch.from_numpy(w).to(torch.bfloat16).to(DEV)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def _check(mats):
    out = woq.ewq_block_entropy(mats, exp_hist=True)
    again = woq.ewq_block_entropy(mats, exp_hist=True)
    h = out["h_mat"].cpu().numpy()
    eh = out["exp_hist"].cpu().numpy()
    assert torch.equal(out["h_mat"].view(torch.int64), again["h_mat"].view(torch.int64))
    assert torch.equal(out["exp_hist"], again["exp_hist"])
    for i, m in enumerate(mats):
        w = m.float().cpu().numpy()
        ref = matrix_entropy(w)
        if np.isnan(ref):
            assert np.isnan(h[i]), i
        else:
            assert abs(h[i] - ref) <= 1e-12 * abs(ref) + 1e-14, (i, h[i], ref)
        assert np.array_equal(eh[i], df11.exponent_histogram(_bits(m))), i
    return out


def test_other_values_in_the_list():
    """A few hundred tiny, subnormal and large values spread over one-unit
    and multi-unit matrices: each unit keeps them in its LDS list and the
    matrix list holds them all."""
    a = _plant(_base(512, 1024, 1), 150, 11, 1e-12, 2e-8)            # one unit
    a = _plant(a, 60, 12, 70.0, 3e4)
    b = _plant(_base(2048, 2048, 2), 1500, 13, 1e-40, 1e-38)          # 8 units, subnormals
    c = _plant(_base(1001, 999, 3), 200, 14, 64.0, 1e3)               # ragged tail, all large
    d = _base(300, 1024, 4)
    d[5, :7] = [0.0, -0.0, 1e-9, -3e-9, 2**-25, -(2**-25), 2**6]      # window edges
    _check([_bf(a), _bf(b), _bf(c), _bf(d)])


def test_zeros_and_non_finite_are_counted_not_listed():
    """Half the weights zero (both signs) and many NaN / inf: counted, so
    no list overflows; entropies with NaN are NaN and the count is exact."""
    z = _base(1024, 1024, 5)
    z[:, ::2] = 0.0
    z[::3, 1::4] = -0.0
    nf = _base(256, 1024, 6)
    nf[:, :300] = np.nan
    nf[7, 300:400] = np.inf
    nf[8, 300:400] = -np.inf
    mats = [_bf(z), _bf(nf)]
    out = _check(mats)
    assert out["nonfinite"].item() == 256 * 300 + 200


def test_unit_list_overflow_spills():
    """More other values in one work unit than its LDS list holds: the
    matrix is recounted from the weights (contiguous and strided)."""
    a = _plant(_base(64, 1024, 7), LDS_LIST + 1, 15, 1e-15, 1e-8)
    big = np.concatenate([_base(96, 1024, 8), _plant(_base(96, 1024, 9), 5000, 16, 100.0, 1e5),
                          _base(96, 1024, 10)], axis=1)
    bt = _bf(big)
    view = bt[:, 1024:2048]                                            # strided, ld = 3072
    assert not view.is_contiguous()
    all_tiny = _bf(_base(128, 512, 11, std=1e-9))                     # every value listed
    _check([_bf(a), view, all_tiny, _bf(_base(16, 64, 12))])


def test_matrix_list_overflow_spills():
    """Units that each keep fewer than 240 other values but together more
    than one matrix's list holds (40 units x 230 > 8192)."""
    rows, cols = 5120, 4096                                            # 40 units
    w = _base(rows, cols, 13)
    rng = np.random.default_rng(17)
    flat = w.reshape(-1)
    for u in range(rows * cols // UNIT):
        pos = u * UNIT + rng.choice(UNIT, size=230, replace=False)
        flat[pos] = rng.uniform(1e-12, 1e-9, size=230)
    assert 40 * 230 > LIST_CAP
    _check([_bf(w), _bf(_plant(_base(512, 1024, 14), 100, 18, 1e-12, 1e-9))])


def test_entropy_many_small_matrices_one_batch():
    """4,704 matrices in one call (the MoE stack's count), small ones and a
    sample of the expert shape: every entropy equals the one-matrix call's
    and the sampled ones the oracle's."""
    n = 4704
    base = _bf(_base(64, 128, 20))
    mats = []
    for i in range(n):
        mats.append(base * (1.0 + 0.001 * (i % 97)) if i % 500 else
                    _bf(_base(1408, 2048, 100 + i, std=0.02 * (1 + i % 3))))
    h = woq.ewq_block_entropy(mats)["h_mat"].cpu().numpy()
    for i in list(range(0, n, 500)) + [1, 2, 97, n - 1]:
        one = woq.ewq_block_entropy([mats[i]])["h_mat"].item()
        assert h[i] == one, i
        ref = matrix_entropy(mats[i].float().cpu().numpy())
        assert abs(h[i] - ref) <= 1e-12 * ref, i
