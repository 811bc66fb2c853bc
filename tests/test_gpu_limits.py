"""The path at its size limits: a matrix just under 2^31 weights at the widest
Sinkhorn row (32768 columns), and the widest rows of both passes' shapes.

The 2^31-weight matrix is a 257 x 4096 block B tiled 255 x 8 (65535 x 32768
= 2,147,450,880 weights, 4.3 GB of bf16).  Tiling fixes the results at any
size without running the oracle on 2^31 weights:
  - entropy: the softmax of k copies of B has entropy H(B) + ln k;
  - Sinkhorn: every row (column) of W repeats a row (column) of B, so s and t
    are B's tiled; equal lines are reduced in the same order, so the tiles
    agree bit for bit;
  - codes (affine and code-book grids): rows are quantised independently,
    so code tiles repeat too;
  - the lossless code: W's exponent histogram is k times B's.
B itself goes through the oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import woqdata
import weight_only_quantization_softmax_amd as woq

pytestmark = pytest.mark.gpu
DEV = "cuda"
RB, CB, KR, KC = 257, 4096, 255, 8


def _np(t):
    return t.detach().float().cpu().numpy()


@pytest.fixture(scope="module")
def tiled():
    b = woqdata.random_matrix(RB, CB, 4242, outlier_frac=0.01, outlier_mult=20.0).to(DEV)
    w = b.repeat(KR, KC)
    assert w.numel() == RB * KR * CB * KC < 2 ** 31
    yield b, w
    del w
    torch.cuda.empty_cache()


def test_entropy_of_a_2_31_matrix(tiled):
    b, w = tiled
    out = woq.ewq_block_entropy([w])
    h = out["h_mat"].item()
    ref = oracle.matrix_entropy(_np(b)) + math.log(KR * KC)
    assert abs(h - ref) <= 1e-10 * ref


def test_sinkhorn_and_codes_of_a_2_31_matrix(tiled):
    b, w = tiled
    s, t = woq.sinq_balance([w], 16)
    s_ref, t_ref = oracle.sinkhorn_std(_np(b), 16)
    sv, tv = s[0].view(KR, RB), t[0].view(KC, CB)
    assert torch.equal(sv, sv[:1].expand_as(sv)) and torch.equal(tv, tv[:1].expand_as(tv))
    np.testing.assert_allclose(sv[0].cpu().numpy(), s_ref, rtol=1e-4)
    np.testing.assert_allclose(tv[0].cpu().numpy(), t_ref, rtol=1e-4)

    codes, scales, zeros = woq.quant_pack_groupwise([w], 4, 64, row_scale=s, col_scale=t)
    c = codes[0].view(KR, RB, KC, CB // 2)
    assert torch.equal(c, c[:1, :, :1].expand_as(c))
    q, d, z = oracle.quantize_groupwise_f32(_np(b), sv[0].cpu().numpy(), tv[0].cpu().numpy(), 4, 64)
    assert np.array_equal(c[0, :, 0].cpu().numpy(), oracle.pack_codes(q, 4))
    dv = scales[0].view(KR, RB, KC, CB // 64)
    assert np.array_equal(dv[0, :, 0].cpu().numpy().view(np.uint32), d.view(np.uint32))
    assert np.array_equal(zeros[0].view(KR, RB, KC, CB // 64)[KR - 1, :, KC - 1].cpu().numpy(), z)

    out = woq.dequant_unpack([tuple(w.shape)], codes, scales, 4, 64, zeros=zeros, row_scale=s,
                             col_scale=t, out_dtype=torch.float32)[0]
    ref = oracle.dequantize_f32(q, d, z, sv[0].cpu().numpy(), tv[0].cpu().numpy(), 64)
    last = out[(KR - 1) * RB:, (KC - 1) * CB:]          # the tile farthest into the buffer
    assert np.array_equal(last.cpu().numpy(), ref)
    del out, codes, scales, zeros

    # the code-book grid on the same matrix: code tiles repeat, the first
    # equals the oracle on B, the last tile decodes exactly
    codes, scales = woq.quant_pack_codebook([w], 4, 64, row_scale=s, col_scale=t)
    c = codes[0].view(KR, RB, KC, CB // 2)
    assert torch.equal(c, c[:1, :, :1].expand_as(c))
    lv = oracle.codebook.normal_levels(4)
    qc, ac = oracle.codebook.quantize_codebook_f32(_np(b), sv[0].cpu().numpy(), tv[0].cpu().numpy(), 4, 64, lv)
    assert np.array_equal(c[0, :, 0].cpu().numpy(), oracle.pack_codes(qc, 4))
    av = scales[0].view(KR, RB, KC, CB // 64)
    assert np.array_equal(av[KR - 1, :, KC - 1].cpu().numpy().view(np.uint32), ac.view(np.uint32))
    out = woq.dequant_codebook([tuple(w.shape)], codes, scales, 4, 64, row_scale=s, col_scale=t)[0]
    ref = oracle.codebook.dequantize_codebook_f32(qc, ac, sv[0].cpu().numpy(), tv[0].cpu().numpy(), 64, lv)
    assert np.array_equal(out[(KR - 1) * RB:, (KC - 1) * CB:].cpu().numpy(), ref)
    del out, codes, scales


def test_lossless_code_of_a_2_31_matrix(tiled):
    b, w = tiled
    hist = woq.df11_exponent_histogram([w]).cpu().numpy()[0].astype(np.int64)
    bits_b = b.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)
    assert np.array_equal(hist, (KR * KC) * oracle.df11.exponent_histogram(bits_b))
    enc = woq.df11_encode([w], [woq.df11_build_code(hist)])
    dec = woq.df11_decode(enc)[0]
    assert torch.equal(dec.view(torch.int16), w.view(torch.int16))
    del enc, dec


WIDE = [((24, 32768), torch.bfloat16), ((9, 32768), torch.float32), ((5, 28672), torch.bfloat16),
        ((3, 32760), torch.bfloat16)]


def test_widest_rows_match_oracle():
    mats = [woqdata.random_matrix(r, c, 60 + i, dtype=dt, outlier_frac=0.01, outlier_mult=20.0).to(DEV)
            for i, ((r, c), dt) in enumerate(WIDE)]
    s, t = woq.sinq_balance(mats, 16)
    for i, m in enumerate(mats):
        s_ref, t_ref = oracle.sinkhorn_std(_np(m), 16)
        np.testing.assert_allclose(s[i].cpu().numpy(), s_ref, rtol=1e-4, err_msg=str(WIDE[i]))
        np.testing.assert_allclose(t[i].cpu().numpy(), t_ref, rtol=1e-4, err_msg=str(WIDE[i]))
    with pytest.raises(woq.WoqError):
        woq.sinq_balance([woqdata.random_matrix(2, 32776, 1).to(DEV)], 1)
