"""GPU parity of the code-book (non-uniform) grid through the C ABI.

Codes and per-group scales are compared bit for bit with the oracle's fp32
decision sequence, fed with the GPU's own balancing scales (stage
isolation); dequantised weights bit for bit (fp32) and after one
round-to-nearest-even (bf16).  Cases cover the three quantise kernels (row
tiles for power-of-two groups up to 512, one wave per group up to 4096
columns, one workgroup per wider group), ragged tiles, zero groups, books
whose midpoints crowd one table cell (several comparisons per value) and
levels outside [-1, 1].  At the size of a Llama-8B block, sampled rows are
compared with the oracle and the whole matrix is checked against the error
bound that holds at any size.
"""
import numpy as np
import pytest
import torch

import woqdata
import weight_only_quantization_softmax_amd as woq
from oracle import codebook as cb
from oracle import rtn

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rm(rows, cols, seed, dtype=torch.bfloat16):
    return woqdata.random_matrix(rows, cols, seed, dtype=dtype, outlier_frac=0.01,
                                 outlier_mult=20.0).to(DEV)


def _np(t):
    return t.detach().float().cpu().numpy()


def _check(m, s, t, bits, group, levels, codes, scales):
    g = group if group else m.shape[1]
    q_ref, a_ref = cb.quantize_codebook_f32(
        _np(m), None if s is None else s.cpu().numpy(), None if t is None else t.cpu().numpy(),
        bits, g, levels)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), a_ref.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), rtn.pack_codes(q_ref, bits))
    return q_ref, a_ref


CASES = [  # (rows, cols, bits, group, dtype)
    (16, 256, 4, 64, torch.bfloat16), (7, 96, 4, 32, torch.bfloat16),
    (33, 384, 3, 128, torch.bfloat16), (9, 512, 2, 8, torch.bfloat16),
    (12, 1024, 4, 512, torch.bfloat16), (256, 512, 4, 64, torch.float32),
    (13, 2560, 4, 64, torch.bfloat16), (11, 1408, 3, 64, torch.float32),
    (10, 1800, 4, 600, torch.bfloat16), (20, 2048, 4, 1024, torch.bfloat16),
    (5, 4096, 3, 0, torch.bfloat16), (4, 3072, 4, 0, torch.float32),
    (4, 16384, 4, 8192, torch.bfloat16), (3, 14336, 4, 0, torch.bfloat16),
    # fp32 groups wider than one wave (one workgroup per group); 2-bit codes
    # over ragged 2048-column tiles
    (3, 8192, 3, 0, torch.float32), (2, 16384, 4, 16384, torch.float32), (11, 2600, 2, 8, torch.bfloat16),
]


@pytest.mark.parametrize("with_scales", [False, True])
def test_codebook_quant_bit_exact(with_scales):
    for i, (r, c, bits, group, dt) in enumerate(CASES):
        print(f"case {i}: {r}x{c} bits={bits} group={group} {dt}", flush=True)
        m = _rm(r, c, 70 + i, dt)
        s = t = None
        if with_scales:
            ss, tt = woq.sinq_balance([m], 3)
            s, t = ss[0], tt[0]
        codes, scales = woq.quant_pack_codebook(
            [m], bits, group, row_scale=None if s is None else [s],
            col_scale=None if t is None else [t])
        _check(m, s, t, bits, group, cb.normal_levels(bits), codes[0], scales[0])


def test_codebook_batched_with_zero_groups():
    mats = [_rm(16, 256, 1), _rm(8, 512, 2, torch.float32), _rm(4, 64, 3),
            torch.zeros(2, 128, device=DEV, dtype=torch.bfloat16)]
    c = torch.full((2, 128), 0.5, device=DEV)
    c[1, 64:] = -0.25
    mats.append(c.to(torch.bfloat16))
    codes, scales = woq.quant_pack_codebook(mats, 4, 64)
    for i, m in enumerate(mats):
        _check(m, None, None, 4, 64, cb.normal_levels(4), codes[i], scales[i])
    # zero groups: a = 0 and every code is the lower of the two levels nearest 0
    assert torch.all(scales[3] == 0)
    assert torch.all(codes[3] == 0x77)


BOOKS = {
    # midpoints crowded into one table cell: several comparisons per value
    "crowded": np.array([-1.0, -0.002, -0.001, 0.0, 0.0005, 0.001, 0.0015, 1.0], dtype=np.float32),
    # levels beyond [-1, 1] and an asymmetric book
    "wide": np.array([-3.0, -0.5, 0.25, 2.0], dtype=np.float32),
    "skewed": np.array([-0.1, 0.0, 0.05, 0.1, 0.2, 0.4, 0.7, 1.0, 1.2, 1.3, 1.4, 1.5, 1.6,
                        1.7, 1.8, 2.5], dtype=np.float32),
}


@pytest.mark.parametrize("name", sorted(BOOKS))
def test_caller_books(name):
    lv = BOOKS[name]
    bits = int(np.log2(lv.size))
    for i, (r, c, group, dt) in enumerate([(16, 256, 64, torch.bfloat16), (10, 1800, 600, torch.float32),
                                           (3, 14336, 0, torch.bfloat16)]):
        m = _rm(r, c, 90 + i, dt)
        ss, tt = woq.sinq_balance([m], 2)
        codes, scales = woq.quant_pack_codebook([m], bits, group, levels=lv.tolist(),
                                                row_scale=ss, col_scale=tt)
        q_ref, a_ref = _check(m, ss[0], tt[0], bits, group, lv, codes[0], scales[0])
        g = group if group else c
        ref = cb.dequantize_codebook_f32(q_ref, a_ref, ss[0].cpu().numpy(), tt[0].cpu().numpy(), g, lv)
        out = woq.dequant_codebook([(r, c)], codes, scales, bits, group, levels=lv.tolist(),
                                   row_scale=ss, col_scale=tt)[0]
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("bits,group,rows,cols", [(4, 64, 24, 1024), (3, 128, 24, 1024),
                                                  (2, 32, 24, 1024), (4, 64, 13, 2560),
                                                  (3, 0, 9, 6144), (4, 600, 5, 1800)])
def test_codebook_dequant_matches_oracle(bits, group, rows, cols):
    m = _rm(rows, cols, 61)
    ss, tt = woq.sinq_balance([m], 2)
    codes, scales = woq.quant_pack_codebook([m], bits, group, row_scale=ss, col_scale=tt)
    g = group if group else cols
    lv = cb.normal_levels(bits)
    q_ref = rtn.unpack_codes(codes[0].cpu().numpy(), bits, cols)
    ref = cb.dequantize_codebook_f32(q_ref, scales[0].cpu().numpy(), ss[0].cpu().numpy(),
                                     tt[0].cpu().numpy(), g, lv)
    out32 = woq.dequant_codebook([(rows, cols)], codes, scales, bits, group, row_scale=ss,
                                 col_scale=tt)[0]
    assert np.array_equal(out32.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    out16 = woq.dequant_codebook([(rows, cols)], codes, scales, bits, group, row_scale=ss,
                                 col_scale=tt, out_dtype=torch.bfloat16)[0]
    assert torch.equal(out16.cpu(), torch.from_numpy(ref).to(torch.bfloat16))


def _error_bound_ok(w, out, s, t, a, g, lv):
    """|W - W'| <= s t a G / 2 (G the widest gap between levels), plus fp32
    rounding, for books spanning [-1, 1]."""
    gap = float(np.max(np.diff(lv.astype(np.float64))))
    bound = np.outer(s, t) * np.repeat(a, g, 1) * (gap / 2)
    return np.all(np.abs(w - out) <= bound * (1 + 1e-4) + 1e-12)


def test_llama8b_block_at_full_size():
    """One Llama-3.1-8B block (q, k, v, o, gate, up, down) balanced and coded
    in one call (4-bit normal book, groups of 64): sampled rows of every
    matrix bit-exact against the oracle, the whole block within the error
    bound, and the fp32 dequantisation bit-exact on the same rows."""
    wl, specs, mats = woqdata.generate("stack8b", device=DEV, blocks=[7])
    ss, tt = woq.sinq_balance(mats, 16)
    codes, scales = woq.quant_pack_codebook(mats, 4, 64, row_scale=ss, col_scale=tt)
    outs = woq.dequant_codebook([tuple(m.shape) for m in mats], codes, scales, 4, 64,
                                row_scale=ss, col_scale=tt)
    torch.cuda.synchronize()
    lv = cb.normal_levels(4)
    for k, m in enumerate(mats):
        r, c = m.shape
        rows = np.unique(np.r_[0, 1, r // 2, r - 2, r - 1,
                              np.random.default_rng(k).integers(0, r, 8)])
        sub = m[rows]
        s_sub = ss[k][rows].cpu().numpy()
        t_np = tt[k].cpu().numpy()
        q_ref, a_ref = cb.quantize_codebook_f32(_np(sub), s_sub, t_np, 4, 64, lv)
        assert np.array_equal(codes[k][rows].cpu().numpy(), rtn.pack_codes(q_ref, 4)), specs[k].name
        assert np.array_equal(scales[k][rows].cpu().numpy().view(np.uint32), a_ref.view(np.uint32))
        ref = cb.dequantize_codebook_f32(q_ref, a_ref, s_sub, t_np, 64, lv)
        assert np.array_equal(outs[k][rows].cpu().numpy().view(np.uint32), ref.view(np.uint32))
        assert _error_bound_ok(_np(m).astype(np.float64), outs[k].cpu().numpy().astype(np.float64),
                               ss[k].cpu().numpy().astype(np.float64), t_np.astype(np.float64),
                               scales[k].cpu().numpy().astype(np.float64), 64, lv), specs[k].name
