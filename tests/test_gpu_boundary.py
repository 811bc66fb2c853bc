"""The C-ABI boundary on the GPU: row-strided matrices, the non-finite weight
count in the workspace head, and the binding's allocations on the call's
stream.

Strided views: the q, k and v column blocks of a fused [d, 3d] projection
(and one of two 14336-column halves, which takes the workgroup form of the
Sinkhorn sweep) give results bit-identical to contiguous copies through
every entry point; a dequantised matrix can be written into a column block
of a larger tensor without touching its other columns.
"""
import numpy as np
import pytest
import torch

import woqdata
import weight_only_quantization_softmax_amd as woq
from weight_only_quantization_softmax_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rm(r, c, seed, dtype=torch.bfloat16):
    return woqdata.random_matrix(r, c, seed, dtype=dtype, outlier_frac=0.01, outlier_mult=20.0).to(DEV)


def _fused():
    """Column slices of fused tensors (row stride ld > cols) and row slices
    (contiguous), with contiguous copies of each."""
    qkv = _rm(1024, 3 * 1024, 1)              # [d, 3d]: q, k, v column blocks, ld = 3072
    gu = _rm(256, 2 * 14336, 2)               # two 14336-column halves, ld = 28672
    f32 = _rm(64, 3 * 512, 3, torch.float32)  # fp32, ld = 1536
    rows = _rm(3 * 512, 1024, 4)              # [3d, d] row blocks: contiguous views
    two = _rm(48, 2 * 8192, 6)                # 8192-column halves (two-wave workgroups), ld = 16384
    views = [qkv[:, :1024], qkv[:, 1024:2048], qkv[:, 2048:], gu[:, 14336:], f32[:, 512:1024],
             two[:, 8192:], rows[512:1024]]
    assert not any(v.is_contiguous() for v in views[:6]) and views[6].is_contiguous()
    return views, [v.contiguous() for v in views]


def _same(a, b):
    if isinstance(a, (list, tuple)):
        return all(_same(x, y) for x, y in zip(a, b))
    if isinstance(a, dict):
        return all(_same(a[k], b[k]) for k in a if k != "nonfinite")
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b)


def test_strided_views_match_contiguous_copies():
    views, copies = _fused()
    assert _same(woq.ewq_block_entropy(views), woq.ewq_block_entropy(copies))
    s_v, t_v = woq.sinq_balance(views, 16)
    s_c, t_c = woq.sinq_balance(copies, 16)
    assert _same(s_v, s_c) and _same(t_v, t_c)
    for bits, group in ((4, 64), (3, 128), (8, 0)):
        a = woq.quant_pack_groupwise(views, bits, group, row_scale=s_v, col_scale=t_v)
        b = woq.quant_pack_groupwise(copies, bits, group, row_scale=s_c, col_scale=t_c)
        assert _same(a, b), (bits, group)
    assert _same(woq.quant_pack_codebook(views, 4, 64, row_scale=s_v, col_scale=t_v),
                 woq.quant_pack_codebook(copies, 4, 64, row_scale=s_c, col_scale=t_c))
    tern = [v for v in views if v.shape[1] <= 16384]
    assert _same(woq.ternary_pack(tern), woq.ternary_pack([c.contiguous() for c in tern]))


def test_dequant_into_a_column_block():
    m = _rm(96, 2048, 5)
    s, t = woq.sinq_balance([m], 4)
    codes, scales, zeros = woq.quant_pack_groupwise([m], 4, 64, row_scale=s, col_scale=t)
    ref = woq.dequant_unpack([(96, 2048)], codes, scales, 4, 64, zeros=zeros, row_scale=s,
                             col_scale=t, out_dtype=torch.bfloat16)[0]
    big = torch.full((96, 3 * 2048), 7.0, dtype=torch.bfloat16, device=DEV)
    out = big[:, 2048:4096]
    woq.dequant_unpack([(96, 2048)], codes, scales, 4, 64, zeros=zeros, row_scale=s, col_scale=t,
                       out_dtype=torch.bfloat16, out=[out])
    assert torch.equal(out, ref)
    assert torch.all(big[:, :2048] == 7.0) and torch.all(big[:, 4096:] == 7.0)


def _plant(m, pos, vals):
    flat = m.view(-1) if m.is_contiguous() else None
    for (r, c), v in zip(pos, vals):
        if flat is not None:
            flat[r * m.shape[1] + c] = v
        else:
            m[r, c] = v


def test_nonfinite_counts():
    """NaN and +-inf weights planted at known positions are counted exactly
    by the entropy call (bf16 histogram, fp32 max pass) and by the first
    Sinkhorn iteration (wave form, workgroup form of four and of two waves,
    fp32, a strided view); a
    row whose squares overflow fp32 without any non-finite weight adds
    nothing; a second call on the same workspace starts from zero."""
    nan, inf = float("nan"), float("inf")
    a = _rm(300, 1024, 11)                     # wave form
    b = _rm(96, 14336, 12)                     # workgroup form
    c = _rm(64, 512, 13, torch.float32)
    big = _rm(128, 3 * 1024, 14)
    d = big[:, 1024:2048]                      # strided view
    e = _rm(32, 1024, 15)
    e[3, 0::2] = 3e38                          # finite weights whose shifted squares overflow
    e[3, 1::2] = -3e38
    f = _rm(40, 8192, 18)                      # workgroup form, two-wave workgroups
    _plant(a, [(0, 0), (7, 1023), (299, 511)], [nan, inf, -inf])
    _plant(f, [(0, 8191), (39, 4096), (17, 0)], [inf, nan, -inf])
    _plant(b, [(5, 14335), (95, 0)], [nan, -inf])
    _plant(c, [(1, 1), (63, 511), (20, 7), (20, 8)], [inf, nan, -inf, nan])
    _plant(d, [(0, 1), (127, 1023)], [inf, nan])
    mats = [a, b, c, d, e, f]
    planted = 3 + 2 + 4 + 2 + 3
    ws = torch.empty(woq.workspace_size(_lib.OP_ENTROPY, mats), dtype=torch.uint8, device=DEV)
    out = woq.ewq_block_entropy(mats, ws=ws)
    assert woq.nonfinite_count(ws).item() == planted
    assert out["nonfinite"].item() == planted
    h = out["h_mat"].cpu().numpy()
    assert np.all(np.isnan(h[:4])) and np.isfinite(h[4]) and np.isnan(h[5])
    for sub, n in (([a], 3), ([b], 2), ([c], 4), ([d], 2), ([e], 0), ([f], 3), (mats, planted)):
        wsq = torch.empty(woq.workspace_size(_lib.OP_SINQ, sub), dtype=torch.uint8, device=DEV)
        wsq.fill_(0xFF)
        woq.sinq_balance(sub, 16, ws=wsq)
        assert woq.nonfinite_count(wsq).item() == n, n
        woq.sinq_balance(sub, 3, ws=wsq)           # the same workspace again
        assert woq.nonfinite_count(wsq).item() == n, n
    wsq = torch.full((woq.workspace_size(_lib.OP_SINQ, [a]),), 0xFF, dtype=torch.uint8, device=DEV)
    woq.sinq_balance([a], 0, ws=wsq)               # no weight read
    assert woq.nonfinite_count(wsq).item() == 0
    clean = [_rm(64, 1024, 16), _rm(64, 14336, 17)]
    ws2 = torch.full((woq.workspace_size(_lib.OP_ENTROPY, clean),), 0xFF, dtype=torch.uint8, device=DEV)
    assert woq.ewq_block_entropy(clean, ws=ws2)["nonfinite"].item() == 0


def test_other_calls_leave_the_head_untouched():
    m = _rm(64, 1024, 21)
    s, t = woq.sinq_balance([m], 2)
    head = torch.arange(_lib.WS_HEAD, dtype=torch.int32, device=DEV).to(torch.uint8)
    for op, call in ((_lib.OP_QUANT, lambda ws: woq.quant_pack_groupwise([m], 4, 64, row_scale=s,
                                                                         col_scale=t, ws=ws)),
                     (_lib.OP_TERNARY, lambda ws: woq.ternary_pack([m], ws=ws)),
                     (_lib.OP_DF11_HIST, lambda ws: woq.df11_exponent_histogram([m], ws=ws))):
        ws = torch.empty(woq.workspace_size(op, [m], 64), dtype=torch.uint8, device=DEV)
        ws[:_lib.WS_HEAD] = head
        call(ws)
        torch.cuda.synchronize()
        assert torch.equal(ws[:_lib.WS_HEAD], head), op


def test_calls_on_a_side_stream_allocate_there():
    """With stream= a side stream and no workspace, the binding allocates the
    workspace and outputs on that stream: memory the main stream then takes
    and overwrites while the side stream still runs cannot be the call's
    workspace, so every result equals the call made alone."""
    mats = [_rm(4096, 4096, 31), _rm(1024, 4096, 32), _rm(2048, 14336, 33)]
    ref_s, ref_t = woq.sinq_balance(mats, 16)
    ref_e = woq.ewq_block_entropy(mats)["h_mat"]
    ref_q = woq.quant_pack_groupwise(mats, 4, 64, row_scale=ref_s, col_scale=ref_t)
    need = max(woq.workspace_size(_lib.OP_SINQ, mats), woq.workspace_size(_lib.OP_QUANT, mats, 64))
    torch.cuda.synchronize()
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    for rep in range(3):
        side.wait_stream(main)
        s, t = woq.sinq_balance(mats, 16, stream=side)
        e = woq.ewq_block_entropy(mats, stream=side)["h_mat"]
        q = woq.quant_pack_groupwise(mats, 4, 64, row_scale=s, col_scale=t, stream=side)
        # the main stream takes memory of the workspace's size and overwrites it
        junk = [torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV) for _ in range(3)]
        main.wait_stream(side)
        torch.cuda.synchronize()
        del junk
        assert _same(s, ref_s) and _same(t, ref_t), rep
        assert torch.equal(e, ref_e), rep
        assert _same(q, ref_q), rep
