"""Pins for the oracle's ternary {-1, 0, +1} per-row-scale quantiser."""
import numpy as np
import torch

import oracle
import woqdata


def test_codes_and_values():
    w = woqdata.random_matrix(32, 256, 3).float().numpy()
    q, beta = oracle.ternary_quantize(w)
    assert set(np.unique(q).tolist()) <= {-1, 0, 1}
    # beta = mean |W| per row (checked with torch's mean/abs)
    ref = torch.from_numpy(w).double().abs().mean(dim=1).float().numpy()
    assert np.array_equal(beta, ref)
    deq = oracle.ternary_dequantize(q, beta)
    for i in range(32):
        assert set(np.unique(deq[i]).tolist()) <= {-beta[i], 0.0, beta[i]}


def test_brute_force_argmin():
    w = woqdata.random_matrix(8, 64, 4).float().numpy()
    q, beta = oracle.ternary_quantize(w)
    for i in range(8):
        for j in range(64):
            errs = {c: abs(float(w[i, j]) - c * float(beta[i])) for c in (-1, 0, 1)}
            best = min(errs.values())
            assert errs[int(q[i, j])] <= best * (1 + 1e-6) + 1e-12


def test_exact_half_rounds_to_zero_and_clamps():
    beta = np.array([1.0], dtype=np.float32)
    w = np.array([[0.5, -0.5, 0.5000001, 1.5, -7.0, 0.0]], dtype=np.float32)
    q, _ = oracle.ternary_quantize(w, beta)
    assert q.tolist() == [[0, 0, 1, 1, -1, 0]]


def test_zero_row():
    w = np.zeros((2, 16), dtype=np.float32)
    w[1, :4] = [0.2, -0.4, 0.0, 0.1]
    q, beta = oracle.ternary_quantize(w)
    assert beta[0] == 0 and np.all(q[0] == 0)
    assert beta[1] == np.float32(np.mean(np.abs(w[1].astype(np.float64))))
    # codes q + 1 pack as 2-bit LSB-first
    packed = oracle.pack_codes((q + 1).astype(np.uint8), 2)
    assert packed.shape == (2, 4) and packed[0].tobytes() == bytes([0x55] * 4)


def test_f64_definition_brute_force():
    # exact rational arithmetic: beta = mean |W|, q = clamp(rne(W / beta))
    from fractions import Fraction
    w = woqdata.random_matrix(6, 64, 5).float().numpy()
    w[2, :] = np.repeat([0.25, -0.5, 0.125, 0.0], 16)   # beta = 0.21875: exact ratios
    w[3, :] = 0.0
    q, beta = oracle.ternary_quantize_f64(w)
    for i in range(6):
        row = [Fraction(float(v)) for v in w[i]]
        b = sum(abs(v) for v in row) / len(row)
        assert beta[i] == float(b) or abs(beta[i] / float(b) - 1) < 1e-15
        for j, v in enumerate(row):
            ref = 0 if b == 0 else min(max(round(v / b), -1), 1)
            assert q[i, j] == ref, (i, j)


def test_near_tie_mask_hand_cases():
    beta = np.array([1.0, 2.0, 0.0])
    w = np.array([[0.5, 0.5 + 2e-5, 0.5 - 5e-6, 1.5, 0.2, -0.5],
                  [1.0, -1.0, 3.0, 1.00004, 0.0, 2.5],
                  [0.5, 0.0, 0.0, 0.0, 0.0, 0.0]])
    m = oracle.ternary_near_tie_mask(w, beta)
    assert m.tolist() == [[True, False, True, True, False, True],
                          [True, True, True, False, False, False],
                          [False] * 6]


def test_f32_decisions_agree_with_f64_except_near_ties():
    w = woqdata.random_matrix(256, 2048, 9).float().numpy()
    q32, b32 = oracle.ternary_quantize(w)
    q64, b64 = oracle.ternary_quantize_f64(w)
    assert np.allclose(b32, b64, rtol=2 ** -24)
    diff = q32 != q64
    assert np.all(~diff | oracle.ternary_near_tie_mask(w))
    assert diff.mean() <= 1e-5
