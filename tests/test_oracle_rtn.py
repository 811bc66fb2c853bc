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
    tie = oracle.near_tie_fraction(w, s, t, d64, z64, 4, 64)
    diff = q32 != q64
    assert np.all(~diff | tie)
    assert np.all(np.abs(q32.astype(int) - q64.astype(int)) <= 1)


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
    tie = oracle.near_tie_fraction(w, None, None, d, z, 8, 4096)
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
