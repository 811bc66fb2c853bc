"""GPU parity of the DF11 lossless exponent code (through the C ABI).

Histogram, encoded buffers (stream, sign/mantissa bytes, gaps, block
positions) and decoded words are compared bit for bit with the oracle on the
same seeded inputs; the decoder is also fed the oracle's own buffers (stage
isolation).  At the full size of a Llama-8B block the property that holds at
any size is checked: decoding returns every bf16 word exactly, and one
projection's stream is compared with the oracle in full.
"""
import numpy as np
import pytest
import torch

import woqdata
import weight_only_quantization_softmax_amd as woq
from oracle import df11

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def _from_bits(b, shape):
    return torch.from_numpy(np.asarray(b, dtype=np.uint16).view(np.int16).copy()).view(
        torch.bfloat16).reshape(shape).to(DEV)


def _check_encoded(t, out):
    bits = _bits(t)
    h = df11.exponent_histogram(bits)
    L, C, T, tot = df11.build_code(h)
    ref = df11.encode(bits, L, C)
    assert out["total_bits"] == tot
    assert np.array_equal(out["enc"].cpu().numpy(), ref["enc"])
    assert np.array_equal(out["sm"].cpu().numpy(), ref["sm"])
    assert np.array_equal(out["gaps"].cpu().numpy(), ref["gaps"])
    assert np.array_equal(out["block_pos"].cpu().numpy().view(np.uint32), ref["block_pos"])
    assert np.array_equal(out["tables"].cpu().numpy().reshape(-1, 256), T)
    return ref, (L, C, T, tot)


SHAPES = [(1, 1), (3, 5), (37, 129), (64, 4096), (300, 1000), (1, 70001)]


@pytest.mark.parametrize("shape", SHAPES)
def test_histogram_encode_decode_match_oracle(shape):
    w = woqdata.random_matrix(shape[0], shape[1], 900 + shape[1], device=DEV)
    hist = woq.df11_exponent_histogram([w]).cpu().numpy()[0]
    assert np.array_equal(hist.astype(np.int64), df11.exponent_histogram(_bits(w)))
    enc = woq.df11_compress([w])
    _check_encoded(w, enc[0])
    out = woq.df11_decode(enc)[0]
    assert torch.equal(out.view(torch.int16), w.view(torch.int16))


def test_batched_matrices_in_one_call():
    shapes = [(128, 512), (7, 9), (256, 1536), (1, 8192), (33, 8193)]
    mats = [woqdata.random_matrix(r, c, 50 + i, std=0.01 * (i + 1), device=DEV)
            for i, (r, c) in enumerate(shapes)]
    enc = woq.df11_compress(mats)
    for m, e in zip(mats, enc):
        _check_encoded(m, e)
    outs = woq.df11_decode(enc)
    for m, o in zip(mats, outs):
        assert torch.equal(o.view(torch.int16), m.view(torch.int16))


def test_decoder_reads_oracle_buffers():
    """Stage isolation: buffers written by the oracle decode on the GPU."""
    w = woqdata.random_matrix(200, 777, 31, device=DEV)
    bits = _bits(w)
    L, C, T, tot = df11.build_code(df11.exponent_histogram(bits))
    ref = df11.encode(bits, L, C)
    e = {"enc": torch.from_numpy(ref["enc"]).to(DEV), "sm": torch.from_numpy(ref["sm"]).to(DEV),
         "gaps": torch.from_numpy(ref["gaps"]).to(DEV),
         "block_pos": torch.from_numpy(ref["block_pos"].view(np.int32)).to(DEV),
         "tables": torch.from_numpy(T.reshape(-1).copy()).to(DEV),
         "code_len": torch.from_numpy(L.astype(np.uint8)).to(DEV),
         "n_tables": T.shape[0], "total_bits": tot, "shape": tuple(w.shape)}
    out = woq.df11_decode([e])[0]
    assert torch.equal(out.view(torch.int16), w.view(torch.int16))


def test_hand_worked_stream_with_an_empty_last_segment():
    exps = np.array([100 + (i % 8) for i in range(22)], dtype=np.uint16)
    bits = (exps << 7).astype(np.uint16)
    w = _from_bits(bits, (2, 11))
    enc = woq.df11_compress([w])[0]
    assert enc["total_bits"] == 66
    assert enc["enc"].cpu().numpy()[:9].tolist() == [5, 57, 119, 5, 57, 119, 5, 57, 64]
    assert enc["gaps"].cpu().numpy().tolist() == [64, 0, 0, 0, 0, 0, 0, 0]
    assert enc["block_pos"].cpu().numpy().tolist() == [0, 22]
    assert torch.equal(woq.df11_decode([enc])[0].view(torch.int16), w.view(torch.int16))


def test_deep_code_with_sub_tables():
    rng = np.random.default_rng(8)
    fib = [1, 1]
    while len(fib) < 24:
        fib.append(fib[-1] + fib[-2])
    exps = rng.permutation(np.repeat(np.arange(60, 84), fib))
    mant = rng.integers(0, 256, exps.size)
    bits = ((mant & 0x80) << 8 | exps << 7 | (mant & 0x7F)).astype(np.uint16)
    n = bits.size - bits.size % 16
    w = _from_bits(bits[:n], (16, n // 16))
    enc = woq.df11_compress([w])[0]
    ref, (L, C, T, tot) = _check_encoded(w, enc)
    assert L.max() > 16 and T.shape[0] >= 3
    assert torch.equal(woq.df11_decode([enc])[0].view(torch.int16), w.view(torch.int16))


def test_segments_with_many_short_codes():
    """Two exponents only: 1-bit codes, up to 64 codes start per segment."""
    rng = np.random.default_rng(9)
    exps = np.where(rng.random(50000) < 0.5, 118, 119)
    bits = (exps << 7 | rng.integers(0, 128, exps.size)).astype(np.uint16)
    w = _from_bits(bits, (100, 500))
    enc = woq.df11_compress([w])[0]
    _check_encoded(w, enc)
    assert torch.equal(woq.df11_decode([enc])[0].view(torch.int16), w.view(torch.int16))


def test_non_codable_exponents_are_rejected():
    w = woqdata.random_matrix(8, 64, 3, device=DEV)
    w[0, 0] = float("inf")
    hist = woq.df11_exponent_histogram([w]).cpu().numpy()[0]
    assert hist[255] == 1
    with pytest.raises(woq.WoqError) as e:
        woq.df11_build_code(hist)
    assert e.value.status == 11


def test_full_llama8b_block_round_trip():
    """One Llama-3.1-8B block (7 matrices, 218M weights) in one batched call:
    every word decodes exactly; k is compared with the oracle in full; the
    size is about 11 bits per weight."""
    wl, specs, mats = woqdata.generate("stack8b", device=DEV, blocks=[5])
    enc = woq.df11_compress(mats)
    torch.cuda.synchronize()
    k = [i for i, s in enumerate(specs) if s.name.endswith(".k")][0]
    _check_encoded(mats[k], enc[k])
    outs = woq.df11_decode(enc)
    torch.cuda.synchronize()
    for m, o in zip(mats, outs):
        assert torch.equal(o.view(torch.int16), m.view(torch.int16))
    n = sum(m.numel() for m in mats)
    nbytes = sum(e["enc"].numel() + e["sm"].numel() + e["gaps"].numel() + 4 * e["block_pos"].numel()
                 + e["tables"].numel() + 256 for e in enc)
    assert 10.3 < 8 * nbytes / n < 11.3


def test_exponent_histograms_from_the_entropy_pass():
    """ewq_block_entropy_ex: each bf16 matrix's exponent histogram, summed
    from the entropy pass's counts (window bins, zeros, NaN / inf, the list
    of other values), equals df11_exponent_histogram's and the oracle's
    (strided views included, fp32 matrices all zero); the entropies are
    those of ewq_block_entropy."""
    import woqdata
    mats = [woqdata.random_matrix(64 + 8 * i, 512, 700 + i, std=0.005 * (1 + i % 4)).to(DEV)
            for i in range(6)]
    big = woqdata.random_matrix(256, 3 * 1024, 710).to(DEV)
    mats += [big[:, 1024:2048], woqdata.random_matrix(33, 64, 711, dtype=torch.float32).to(DEV)]
    mats[0][3, :5] = torch.tensor([0.0, -0.0, 1e-30, 3e5, -7e4], device=DEV).to(torch.bfloat16)
    out = woq.ewq_block_entropy(mats, exp_hist=True)
    ref = woq.ewq_block_entropy(mats)
    assert torch.equal(out["h_mat"], ref["h_mat"])
    eh = out["exp_hist"].cpu().numpy()
    bf = [m for m in mats if m.dtype == torch.bfloat16]
    dh = woq.df11_exponent_histogram([m.contiguous() for m in bf]).cpu().numpy()
    for i, m in enumerate(mats):
        if m.dtype == torch.float32:
            assert not eh[i].any()
            continue
        bits = m.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
        assert np.array_equal(eh[i], df11.exponent_histogram(bits)), i
        assert np.array_equal(eh[i], dh[i]), i
