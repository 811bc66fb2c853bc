"""Pins of the DFloat11-style codec oracle (CPU only).

The oracle is checked against things other than itself: a textbook Huffman
example, brute force over all code-length vectors on small alphabets,
hand-worked streams (tests/golden/df11_small.json), an independent
bit-by-bit decoder, the Shannon bound against the closed-form exponent
entropy of Gaussian weights, and the page's own size and table-count
figures.
"""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.stats import norm

from oracle import df11

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "df11_small.json")))


def _hist(symbols, counts):
    h = np.zeros(256, dtype=np.int64)
    h[list(symbols)] = counts
    return h


def _cost(h, lens):
    return int(np.sum(np.asarray(h) * np.asarray(lens)))


def _brute_min_cost(weights, max_len):
    """Least sum w*l over all length vectors with l_i <= max_len and
    Kraft sum 2^-l_i <= 1 (exact integer arithmetic)."""
    n = len(weights)
    best = None
    for ls in itertools.product(range(1, max_len + 1), repeat=n):
        if sum(1 << (max_len - l) for l in ls) <= (1 << max_len):
            c = sum(w * l for w, l in zip(weights, ls))
            best = c if best is None else min(best, c)
    return best


# ------------------------------------------------------------- code lengths
def test_huffman_textbook_example():
    g = GOLD["clrs_huffman"]
    h = _hist(g["symbols"], g["counts"])
    lens = df11.huffman_lengths(h)
    assert [int(lens[s]) for s in g["symbols"]] == g["lengths"]
    assert _cost(h, lens) == g["cost"]


@pytest.mark.parametrize("seed", range(12))
def test_huffman_and_package_merge_optimal_by_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 7))
    w = [int(x) for x in rng.integers(1, 60, n)]
    if seed % 3 == 0:
        w = [1 << i for i in range(n)]          # skewed: the deepest tree
    h = _hist(range(50, 50 + n), w)
    lh = df11.huffman_lengths(h)
    assert _cost(h, lh) == _brute_min_cost(w, n - 1)
    for L in range(max(1, int(np.ceil(np.log2(n)))), n):
        lp = df11.package_merge_lengths(h, L)
        used = lp[50:50 + n]
        assert used.max() <= L and np.sum(2.0 ** -used) <= 1.0
        assert _cost(h, lp) == _brute_min_cost(w, L), (w, L)


def test_length_limit_engages_on_deep_trees():
    # Fibonacci counts make Huffman's tree a path: depth n - 1 = 39 > 32.
    fib = [1, 1]
    while len(fib) < 40:
        fib.append(fib[-1] + fib[-2])
    h = _hist(range(100, 140), fib)
    lh = df11.huffman_lengths(h)
    assert lh.max() == 39
    lens = df11.code_lengths(h)
    assert lens.max() == 32 and np.sum(2.0 ** -lens[lens > 0]) == 1.0
    # package-merge with room for the full depth is optimal, hence as cheap as Huffman
    assert _cost(h, df11.package_merge_lengths(h, 39)) == _cost(h, lh)
    assert _cost(h, lens) >= _cost(h, lh)
    # limiting costs little here (the rare exponents are rare)
    assert _cost(h, lens) <= _cost(h, lh) * 1.0001


def test_canonical_codes_are_a_complete_prefix_code():
    rng = np.random.default_rng(7)
    h = np.zeros(256, dtype=np.int64)
    h[90:135] = rng.integers(1, 10**6, 45)
    lens = df11.code_lengths(h)
    codes = df11.canonical_codes(lens)
    words = [format(int(codes[s]), "0%db" % int(lens[s])) for s in range(256) if lens[s]]
    for a, b in itertools.permutations(words, 2):
        assert not b.startswith(a)
    assert sum(2.0 ** -len(wd) for wd in words) == 1.0
    # canonical: ordered by (length, exponent), code values increase
    order = sorted((int(lens[s]), s) for s in range(256) if lens[s])
    vals = [int(codes[s]) << (32 - L) for L, s in order]
    assert vals == sorted(vals) and len(set(vals)) == len(vals)


def test_degenerate_alphabets():
    h = _hist([127], [5])
    lens, codes, tabs, total = df11.build_code(h)
    assert lens[127] == 1 and codes[127] == 0 and total == 5
    assert np.all(tabs[0][:128] == 127)
    lens, codes, tabs, total = df11.build_code(np.zeros(256, dtype=np.int64))
    assert total == 0 and lens.max() == 0 and tabs.shape == (1, 256)
    assert df11.sizes(0) == (0, 8, 4, 0)


def test_exponents_used_as_pointers_are_rejected():
    h = _hist([120, 255], [10, 1])          # 255: inf / NaN
    with pytest.raises(df11.DF11Error):
        df11.build_code(h)
    h = _hist([120, 240], [10, 1])          # |x| >= 2^113
    with pytest.raises(df11.DF11Error):
        df11.build_code(h)


# ---------------------------------------------------------------- encoding
def test_hand_worked_three_symbols():
    g = GOLD["three_symbols"]
    bits = np.array(g["bits"], dtype=np.uint16)
    h = df11.exponent_histogram(bits)
    lens, codes, tabs, total = df11.build_code(h)
    for s, L in g["lengths"].items():
        assert lens[int(s)] == L and codes[int(s)] == g["codes"][s]
    assert total == g["total_bits"]
    for lo, hi, v in g["root_runs"]:
        assert np.all(tabs[0][lo:hi] == v)
    e = df11.encode(bits, lens, codes)
    assert e["enc"].size == g["enc_bytes"]
    assert e["enc"][:len(g["enc_prefix"])].tolist() == g["enc_prefix"]
    assert not e["enc"][len(g["enc_prefix"]):].any()
    assert e["sm"].tolist() == g["sm"]
    assert e["gaps"].tolist() == g["gaps"] and e["block_pos"].tolist() == g["block_pos"]


def test_hand_worked_segment_without_a_code_start():
    g = GOLD["eight_symbols_two_segments"]
    bits = (np.array(g["exponents"], dtype=np.uint16) << 7).astype(np.uint16)
    lens, codes, tabs, total = df11.build_code(df11.exponent_histogram(bits))
    assert all(lens[e] == 3 and codes[e] == e - 100 for e in range(100, 108))
    e = df11.encode(bits, lens, codes)
    assert total == g["total_bits"] == e["total_bits"]
    assert e["enc"].size == g["enc_bytes"] and e["gaps"].size == g["gap_bytes"]
    assert e["enc"][:9].tolist() == g["enc_prefix"] and not e["enc"][9:].any()
    assert e["gaps"].tolist() == g["gaps"] and e["block_pos"].tolist() == g["block_pos"]
    out = df11.decode_tables(e["enc"], e["gaps"], e["block_pos"], tabs, lens, total, e["sm"])
    assert np.array_equal(out, bits)


def _gauss_bits(n, seed, std=0.02):
    x = np.random.default_rng(seed).normal(0, std, n).astype(np.float32)
    u = x.view(np.uint32)
    # round to nearest even bf16 (integer form of the IEEE rule)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r


@pytest.mark.parametrize("n,seed", [(1, 0), (37, 1), (5000, 2), (40000, 3)])
def test_round_trip_two_decoders(n, seed):
    bits = _gauss_bits(n, seed)
    lens, codes, tabs, total = df11.build_code(df11.exponent_histogram(bits))
    e = df11.encode(bits, lens, codes)
    n_seg, eb, gb, nb = df11.sizes(total)
    assert (e["enc"].size, e["gaps"].size, e["block_pos"].size) == (eb, gb, nb + 1)
    seq = df11.decode_sequential(e["enc"], total, lens, codes, e["sm"])
    assert np.array_equal(seq, bits)
    tab = df11.decode_tables(e["enc"], e["gaps"], e["block_pos"], tabs, lens, total, e["sm"])
    assert np.array_equal(tab, bits)


def test_round_trip_deep_code_uses_sub_tables():
    # exponents with Fibonacci counts: codes up to 32 bits, several sub-tables
    # (exact Fibonacci counts over 21 exponents: a path of depth 20)
    fib = [1, 1]
    while len(fib) < 21:
        fib.append(fib[-1] + fib[-2])
    rng = np.random.default_rng(4)
    exps = rng.permutation(np.repeat(np.arange(60, 81), fib))
    mant = rng.integers(0, 256, exps.size)
    bits = ((mant & 0x80) << 8 | exps << 7 | (mant & 0x7F)).astype(np.uint16)
    lens, codes, tabs, total = df11.build_code(df11.exponent_histogram(bits))
    assert lens.max() > 16 and len(tabs) >= 3
    e = df11.encode(bits, lens, codes)
    out = df11.decode_tables(e["enc"], e["gaps"], e["block_pos"], tabs, lens, total, e["sm"])
    assert np.array_equal(out, bits)


def test_gaps_and_block_positions_follow_their_definitions():
    bits = _gauss_bits(70000, 5)
    lens, codes, _, total = df11.build_code(df11.exponent_histogram(bits))
    e = df11.encode(bits, lens, codes)
    L = lens[(bits >> 7) & 0xFF].astype(np.int64)
    starts = np.cumsum(L) - L
    gb = np.unpackbits(e["gaps"], bitorder="little")
    n_seg = e["n_seg"]
    gaps = np.array([sum(int(gb[5 * t + k]) << k for k in range(5)) for t in range(n_seg)])
    for t in range(n_seg):
        ins = starts[(starts >= 64 * t)]
        first = ins[0] if ins.size else total
        assert gaps[t] == first - 64 * t <= 31
    assert e["n_blocks"] >= 2
    for b in range(e["n_blocks"]):
        assert e["block_pos"][b] == np.count_nonzero(starts < 16384 * b)
    assert e["block_pos"][-1] == bits.size


# -------------------------------------------------------------------- sizes
def test_gaussian_exponent_entropy_and_size_match_the_page():
    """Closed form: for w ~ N(0, s^2) the exponent k = floor(log2 |w|) has
    P(k) = 2 (Phi(2^(k+1)/s) - Phi(2^k/s)); its entropy is about 2.55 bits
    (the page: about 2.6 bits of the 8).  Huffman's mean length lies in
    [H, H + 1) (Shannon), and the whole format comes to about 11 bits per
    weight (the page: about 11 bits, 70% of bf16) with 4 to 8 tables at the
    size of a 4096 x 4096 projection (Gaussian tails are lighter than real
    weights, so smaller samples need fewer tables)."""
    s = 0.02
    ks = np.arange(-140, 4)
    P = 2 * (norm.cdf(2.0 ** (ks + 1) / s) - norm.cdf(2.0 ** ks / s))
    P = P[P > 0]
    H = float(-(P * np.log2(P)).sum())
    assert 2.5 < H < 2.65
    bits = _gauss_bits(1 << 24, 6, std=s)     # about one 4096 x 4096 projection
    h = df11.exponent_histogram(bits)
    p = h[h > 0] / h.sum()
    H_emp = float(-(p * np.log2(p)).sum())
    assert abs(H_emp - H) < 0.01
    lens, codes, tabs, total = df11.build_code(h)
    mean = total / h.sum()
    assert H_emp <= mean < H_emp + 1
    n_seg, eb, gb, nb = df11.sizes(total)
    bpw = (8 * h.sum() + 8 * eb + 8 * gb + 32 * (nb + 1)) / h.sum()
    assert 10.5 < bpw < 11.2
    assert 4 <= len(tabs) <= 8
