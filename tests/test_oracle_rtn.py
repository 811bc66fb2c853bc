"""Pins for the oracle's group RTN quantiser, bit packing and dequantiser."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import rtn
from tests import _brute
import woqdata

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_bit_patterns():
    g = json.load(open(os.path.join(GOLD, "pack_bits.json")))
    for case in g["cases"]:
        q = np.array([case["codes"]], dtype=np.uint8)
        packed = oracle.pack_codes(q, case["bits"])
        assert packed.tobytes().hex() == case["hex"], case
        back = oracle.unpack_codes(packed, case["bits"], q.shape[1])
        assert np.array_equal(back, q)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_round_trip_bijection(bits):
    rng = np.random.default_rng(bits)
    q = rng.integers(0, 2 ** bits, size=(7, 64), dtype=np.uint8)
    p = oracle.pack_codes(q, bits)
    assert p.shape == (7, 64 * bits // 8)
    assert np.array_equal(oracle.unpack_codes(p, bits, 64), q)
    # distinct code rows give distinct byte rows
    q2 = q.copy()
    q2[3, 17] ^= 1
    assert not np.array_equal(oracle.pack_codes(q2, bits), p)


def _bal(seed, rows=16, cols=256):
    w = woqdata.random_matrix(rows, cols, seed).float().numpy()
    s, t = oracle.sinkhorn_std(w, 4)
    return w, s.astype(np.float32), t.astype(np.float32)


@pytest.mark.parametrize("bits,group", [(4, 64), (3, 128), (8, 256), (2, 32), (4, 256)])
def test_codes_in_range_and_error_bound_f64(bits, group):
    w, s, t = _bal(bits * 10 + group)
    q, d, z = oracle.quantize_groupwise_f64(w, s, t, bits, group)
    assert q.max() <= 2 ** bits - 1 and z.max() <= 2 ** bits - 1
    x = w.astype(np.float64) / np.outer(s.astype(np.float64), t.astype(np.float64))
    rec = (q.astype(np.float64) - np.repeat(z, group, 1)) * np.repeat(d, group, 1)
    assert np.all(np.abs(x - rec) <= np.repeat(d, group, 1) / 2 * (1 + 1e-12))


@pytest.mark.parametrize("bits,group", [(4, 64), (3, 128), (8, 64)])
def test_f32_error_bound_with_ulp_slack(bits, group):
    w, s, t = _bal(bits + group)
    q, d, z = oracle.quantize_groupwise_f32(w, s, t, bits, group)
    x = rtn.balanced_f32(w, s, t).astype(np.float64)
    rec = (q.astype(np.float64) - np.repeat(z, group, 1)) * np.repeat(d, group, 1).astype(np.float64)
    dd = np.repeat(d, group, 1).astype(np.float64)
    assert np.all(np.abs(x - rec) <= dd / 2 + 1e-5 * dd)


def test_brute_force_argmin():
    w, s, t = _bal(11, rows=4, cols=64)
    for bits, group in [(4, 64), (3, 32), (2, 16)]:
        q, d, z = oracle.quantize_groupwise_f64(w, s, t, bits, group)
        x = w.astype(np.float64) / np.outer(s.astype(np.float64), t.astype(np.float64))
        for i in range(4):
            for k in range(64 // group):
                seg = x[i, k * group:(k + 1) * group]
                best = _brute.rtn_argmin_codes(seg, d[i, k], z[i, k], 2 ** bits - 1)
                for j, b in enumerate(best):
                    assert int(q[i, k * group + j]) in b


def test_f32_and_f64_agree_except_near_ties():
    w, s, t = _bal(21, rows=64, cols=512)
    q32, d32, z32 = oracle.quantize_groupwise_f32(w, s, t, 4, 64)
    q64, d64, z64 = oracle.quantize_groupwise_f64(w, s, t, 4, 64)
    assert np.allclose(d32, d64, rtol=1e-6)
    tie = oracle.near_tie_mask(w, s, t, 4, 64)
    diff = q32 != q64
    assert np.all(~diff | tie)
    assert np.all(np.abs(q32.astype(int) - q64.astype(int)) <= 1)


def test_near_tie_mask_hand_cases():
    # bits 4 (2^b - 1 = 15), groups of 8; every group spans hi - lo = 15, so
    # u = x / delta = x and the zero-point ratio is -lo.
    w = np.array([
        # lo = 0: z ratio 0 (no tie).  Exact halves flag; +-2e-5 away does not;
        # an integer (6.0) is not a tie; 5e-6 from a half is.
        [0.0, 15.0, 2.5, 3.5 + 2e-5, 7.25, 4.5 - 2e-5, 6.0, 5.5 + 5e-6],
        # lo = -3 (z ratio 3, no tie): negative halves flag as well
        [-3.0, 12.0, -2.5, -1.5 - 2e-5, 0.5, 1.0, -0.25, 11.5],
        # lo = -1.5: the zero-point ratio 1.5 is a tie, so the whole group is
        [-1.5, 13.5, 0.3, 1.0, 2.0, 3.7, 4.1, 5.2],
    ])
    m = oracle.near_tie_mask(w, None, None, 4, 8)
    assert m.tolist() == [
        [False, False, True, False, False, False, False, True],
        [False, False, True, False, True, False, False, True],
        [True] * 8,
    ]
    # scales enter through x = w / (s t): doubling s and w leaves the mask
    s2 = np.full(3, 2.0)
    assert np.array_equal(oracle.near_tie_mask(2 * w, s2, None, 4, 8), m)
    # a group of zeros (span 0) has no rounding at all
    assert not oracle.near_tie_mask(np.zeros((1, 8)), None, None, 4, 8).any()


def test_near_tie_rate_on_a_balanced_bf16_matrix():
    # After balancing, x / delta has no lattice structure, so a fraction
    # close to 2 eps of the elements lies within eps of a half-way point
    # (element ties), and a fraction close to 2 eps of the groups has a
    # near-tie zero-point.  A mask that is too permissive (a larger eps, the
    # distance to the nearest integer instead of the nearest half) or that
    # misses the group rule fails these bounds.
    w = woqdata.random_matrix(1024, 4096, 7).float().numpy()
    s, t = oracle.sinkhorn_std(w, 4)
    eps = 1e-5
    m = oracle.near_tie_mask(w, s, t, 4, 64, eps)
    me = oracle.near_tie_mask(w, s, t, 4, 64, eps) & ~_zero_point_tie(w, s, t, 4, 64, eps)
    n = w.size
    assert 0.6 * 2 * eps < me.sum() / n < 1.5 * 2 * eps
    assert m.sum() / n < 2e-4
    groups = _zero_point_tie(w, s, t, 4, 64, eps).reshape(1024, 64, 64)[:, :, 0]
    # the whole group of a zero-point tie is flagged
    assert np.all(m.reshape(1024, 64, 64)[groups])


def _zero_point_tie(w, s, t, bits, group, eps):
    """Reference for the group rule in plain loops over the groups."""
    x = np.asarray(w, np.float64) / np.outer(np.asarray(s, np.float64), np.asarray(t, np.float64))
    qmax = 2 ** bits - 1
    out = np.zeros(x.shape, bool)
    for i in range(x.shape[0]):
        for k in range(x.shape[1] // group):
            g = x[i, k * group:(k + 1) * group]
            lo, hi = min(0.0, g.min()), max(0.0, g.max())
            if hi > lo:
                uz = qmax * -lo / (hi - lo)
                if abs(uz - np.floor(uz) - 0.5) < eps:
                    out[i, k * group:(k + 1) * group] = True
    return out


def _exact_codes(x, bits, group):
    """The definition in exact rational arithmetic: delta = (hi - lo) / qmax,
    z = rne(-lo / delta), q = clamp(rne(x / delta) + z); Python's round() of a
    Fraction rounds half to even."""
    from fractions import Fraction
    qmax = 2 ** bits - 1
    rows, cols = x.shape
    q = np.zeros((rows, cols), np.int64)
    z = np.zeros((rows, cols // group), np.int64)
    for i in range(rows):
        for k in range(cols // group):
            g = [Fraction(float(v)) for v in x[i, k * group:(k + 1) * group]]
            lo, hi = min(Fraction(0), min(g)), max(Fraction(0), max(g))
            if hi == lo:
                continue
            d = (hi - lo) / qmax
            zk = min(max(round(-lo / d), 0), qmax)
            z[i, k] = zk
            for j, v in enumerate(g):
                q[i, k * group + j] = min(max(round(v / d) + zk, 0), qmax)
    return q, z


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 16), (3, 8), (2, 8)])
def test_f64_decides_exact_half_way_points(bits, group):
    # bf16 values on a coarse lattice (small integers times a power of two)
    # and symmetric groups make many ratios exact half-way points; the fp64
    # definition must round every one of them as exact arithmetic does.
    rng = np.random.default_rng(bits * 100 + group)
    x = rng.integers(-24, 25, size=(6, 4 * group)).astype(np.float64) * 2.0 ** -7
    x[0, :group] = np.linspace(-1, 1, group)       # hi = -lo: z ratio = qmax / 2
    x[1, group - 1] = -x[1, :group - 1].max()      # another symmetric group
    x = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    q_ref, z_ref = _exact_codes(x, bits, group)
    q, d, z = oracle.quantize_groupwise_f64(x, None, None, bits, group)
    assert np.array_equal(z.astype(np.int64), z_ref)
    assert np.array_equal(q.astype(np.int64), q_ref)
    # the fixture does contain exact ties, in the elements and the zero-points
    assert oracle.near_tie_mask(x, None, None, bits, group, 1e-12).sum() >= group


def test_zero_delta_groups():
    w = np.zeros((2, 128), dtype=np.float32)
    w[1, 64:] = 0.5   # constant positive group: lo = 0, hi = 0.5 (not degenerate)
    q, d, z = oracle.quantize_groupwise_f32(w, None, None, 4, 64)
    assert d[0, 0] == 0 and d[0, 1] == 0 and d[1, 0] == 0
    assert np.all(q[0] == 0) and np.all(q[1, :64] == 0) and z[0, 0] == 0
    assert d[1, 1] == np.float32(0.5) / np.float32(15)
    assert np.all(q[1, 64:] == 15) and z[1, 1] == 0
    # tiny subnormal range whose reciprocal overflows counts as degenerate
    w2 = np.zeros((1, 64), dtype=np.float32)
    w2[0, 3] = np.float32(1e-44)
    q2, d2, z2 = oracle.quantize_groupwise_f32(w2, None, None, 4, 64)
    assert np.all(q2 == 0) and z2[0, 0] == 0


def test_int8_per_row_matches_torch_affine():
    # PyTorch's documented affine map q = clamp(round(x / scale) + zero_point)
    w = woqdata.random_matrix(8, 4096, 31).float().numpy()
    q, d, z = oracle.quantize_groupwise_f32(w, None, None, 8, 4096)
    tq = torch.quantize_per_channel(torch.from_numpy(w), torch.from_numpy(d[:, 0].astype(np.float64)),
                                    torch.from_numpy(z[:, 0].astype(np.int64)), 0, torch.quint8)
    tqi = tq.int_repr().numpy()
    tie = oracle.near_tie_mask(w, None, None, 8, 4096)
    diff = tqi != q
    assert np.all(~diff | tie)
    assert diff.mean() < 1e-3


def test_dequant_round_trip_bound():
    w, s, t = _bal(41, rows=32, cols=256)
    q, d, z = oracle.quantize_groupwise_f32(w, s, t, 4, 64)
    rec = oracle.dequantize_f32(q, d, z, s, t, 64).astype(np.float64)
    bound = np.outer(s, t) * np.repeat(d, 64, 1) / 2
    assert np.all(np.abs(w - rec) <= bound * (1 + 1e-4) + 1e-12)


def test_shape_validation():
    with pytest.raises(ValueError):
        oracle.quantize_groupwise_f32(np.zeros((2, 100), np.float32), None, None, 4, 64)
    with pytest.raises(ValueError):
        oracle.quantize_groupwise_f32(np.zeros((2, 64), np.float32), None, None, 5, 64)
    with pytest.raises(ValueError):
        oracle.pack_codes(np.zeros((1, 3), np.uint8), 3)
