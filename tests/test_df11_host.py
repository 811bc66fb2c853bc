"""DF11 host side through the C ABI (CPU only): the native code builder
against the oracle, buffer sizes, and argument checks that must reject
before any HIP call."""
import ctypes
import json
import os

import numpy as np
import pytest

import weight_only_quantization_softmax_amd as woq
from oracle import df11
from weight_only_quantization_softmax_amd import _lib

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libwoq.so not built")
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "df11_small.json")))
FAKE = 0x10000


def _fib(k):
    f = [1, 1]
    while len(f) < k:
        f.append(f[-1] + f[-2])
    return f[:k]


def _random_hists(n, seed):
    rng = np.random.default_rng(seed)
    for trial in range(n):
        h = np.zeros(256, dtype=np.int64)
        k = int(rng.integers(1, 60))
        lo = int(rng.integers(0, 240 - k))
        if trial % 5 == 0:                     # deep trees (some beyond 32 bits)
            kk = min(k, 45)
            h[lo:lo + kk] = _fib(kk)
        else:
            h[lo:lo + k] = rng.integers(0, 10 ** int(rng.integers(1, 9)), k)
            if h.sum() == 0:
                h[lo] = 1
        yield h


def test_native_code_builder_matches_oracle():
    limited = 0
    for h in _random_hists(300, 11):
        L, C, T, tot = df11.build_code(h)
        c = woq.df11_build_code(h)
        assert np.array_equal(c["code_len"], L)
        assert np.array_equal(c["codeword"], C)
        assert np.array_equal(c["tables"], T)
        assert c["total_bits"] == tot
        limited += int(df11.huffman_lengths(h).max() > 32)
    assert limited > 5      # the length-limited path was exercised


def test_native_code_builder_hand_examples():
    g = GOLD["clrs_huffman"]
    h = np.zeros(256, dtype=np.int64)
    h[g["symbols"]] = g["counts"]
    c = woq.df11_build_code(h)
    assert [int(c["code_len"][s]) for s in g["symbols"]] == g["lengths"]
    assert c["total_bits"] == g["cost"]
    g = GOLD["three_symbols"]
    h = np.zeros(256, dtype=np.int64)
    h[[120, 121, 122]] = [2, 1, 1]
    c = woq.df11_build_code(h)
    for s, L in g["lengths"].items():
        assert c["code_len"][int(s)] == L and c["codeword"][int(s)] == g["codes"][s]
    for lo, hi, v in g["root_runs"]:
        assert np.all(c["tables"][0][lo:hi] == v)


def test_native_code_builder_errors():
    h = np.zeros(256, dtype=np.int64)
    h[[100, 255]] = [5, 1]
    with pytest.raises(woq.WoqError) as e:
        woq.df11_build_code(h)
    assert e.value.status == 11
    h = np.zeros(256, dtype=np.int64)
    h[100] = -1
    with pytest.raises(woq.WoqError) as e:
        woq.df11_build_code(h)
    assert e.value.status == 2
    c = woq.df11_build_code(np.zeros(256, dtype=np.int64))
    assert c["total_bits"] == 0 and c["tables"].shape == (1, 256)


@pytest.mark.parametrize("n,bits", [(1, 1), (22, 66), (100, 320), (10**6, 2600000), (5, 160)])
def test_buffer_sizes_match_oracle(n, bits):
    n_seg, eb, gb, nb = df11.sizes(bits)
    assert woq.df11_buffer_sizes(n, bits) == (n_seg, eb, gb, nb)


def test_buffer_sizes_reject_impossible_totals():
    for n, bits in ((10, 9), (10, 321), (0, 0)):
        with pytest.raises(woq.WoqError):
            woq.df11_buffer_sizes(n, bits)


def _code_arrays(lens, cws):
    cl = np.ascontiguousarray(lens, dtype=np.uint8)
    cw = np.ascontiguousarray(cws, dtype=np.uint32)
    a = (ctypes.c_void_p * 1)(cl.ctypes.data)
    b = (ctypes.c_void_p * 1)(cw.ctypes.data)
    return cl, cw, ctypes.cast(a, _lib.PP), ctypes.cast(b, _lib.PP)


def test_encode_and_decode_reject_on_the_host():
    lib = _lib.load()
    m = _lib.mat_array([(FAKE, _lib.WOQ_BF16, 16, 64)])
    mf = _lib.mat_array([(FAKE, _lib.WOQ_F32, 16, 64)])
    ptrs = _lib.ptr_array([FAKE])
    lens = np.zeros(256, dtype=np.uint8)
    cws = np.zeros(256, dtype=np.uint32)
    lens[[120, 121, 122]] = [1, 2, 2]
    cws[[120, 121, 122]] = [0, 2, 3]
    keep = _code_arrays(lens, cws)
    tb = (ctypes.c_int64 * 1)(2048)

    def enc(mats, code, total, ws=FAKE, wsb=1 << 30):
        return lib.df11_encode(mats, 1, code[2], code[3], total, ptrs, ptrs, ptrs, ptrs,
                               ws, wsb, None)
    assert enc(mf, keep, tb) == 3                                   # dtype
    assert enc(m, keep, (ctypes.c_int64 * 1)(1023)) == 2            # total < n
    assert enc(m, keep, (ctypes.c_int64 * 1)(32 * 1024 + 1)) == 2   # total > 32 n
    bad = lens.copy()
    bad[123] = 1                                                     # Kraft sum > 1
    assert enc(m, _code_arrays(bad, cws), tb) == 11
    bad = lens.copy()
    bad[250] = 3                                                     # pointer exponent
    assert enc(m, _code_arrays(bad, cws), tb) == 11
    badcw = cws.copy()
    badcw[120] = 2                                                   # codeword wider than its length
    assert enc(m, _code_arrays(lens, badcw), tb) == 11
    assert enc(m, keep, tb, ws=FAKE + 16) == 6                       # misaligned workspace
    assert enc(m, keep, tb, wsb=64) == 6                             # workspace too small

    nt = (ctypes.c_int32 * 1)(0)

    def dec(mats, ntab, total, p=ptrs):
        return lib.df11_decode(mats, 1, p, p, p, p, p, ntab, p, total, FAKE, 1 << 30, None)
    assert dec(m, nt, tb) == 2                                       # no tables
    assert dec(m, (ctypes.c_int32 * 1)(18), tb) == 2                 # too many tables
    assert dec(mf, (ctypes.c_int32 * 1)(3), tb) == 3
    assert dec(m, (ctypes.c_int32 * 1)(3), (ctypes.c_int64 * 1)(5)) == 2
    assert dec(m, (ctypes.c_int32 * 1)(3), tb, p=_lib.ptr_array([None])) == 1
    h = (ctypes.c_int64 * 1)(0)
    assert lib.df11_exponent_histogram(mf, 1, FAKE, FAKE, 1 << 30, None) == 3
    assert lib.df11_exponent_histogram(m, 1, None, FAKE, 1 << 30, None) == 1
    assert lib.df11_exponent_histogram(m, 1, FAKE + 4, FAKE, 1 << 30, None) == 9
    del h


def test_workspace_sizes_for_df11_ops():
    m = _lib.mat_array([(FAKE, _lib.WOQ_BF16, 1000, 60)])     # any width
    for op in (_lib.OP_DF11_HIST, _lib.OP_DF11_ENCODE, _lib.OP_DF11_DECODE):
        out = ctypes.c_size_t(0)
        assert _lib.load().woq_workspace_size(op, m, 1, 0, ctypes.byref(out)) == 0
        assert out.value > 0
