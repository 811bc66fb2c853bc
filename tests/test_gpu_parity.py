"""GPU parity: every entry point through the C ABI against the CPU oracle.

Bars: entropies within 1e-5 relative (the kernels reach ~1e-12); Sinkhorn
scales within 1e-4 relative; codes, deltas and zero-points bit-exact against
the oracle's fp32 decision sequence fed with the GPU's own upstream scales
(stage isolation); against the plain fp64 definition (the GPU's scales),
code differences are allowed only at near ties, by one, and must be <= 1e-5
of all elements; end to end (the oracle's own scales) by one, <= 1e-5.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import woqdata
import weight_only_quantization_softmax_amd as woq
from tests import _codes

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rm(rows, cols, seed, dtype=torch.bfloat16, std=0.02, frac=0.001, mult=10.0):
    return woqdata.random_matrix(rows, cols, seed, dtype=dtype, std=std, outlier_frac=frac,
                                 outlier_mult=mult).to(DEV)


def _np(t):
    return t.detach().float().cpu().numpy() if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


# ------------------------------------------------------------------ entropy
ENT_SHAPES = [(3, 5), (1, 8), (64, 100), (257, 1000), (1024, 1536), (2, 700001)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_entropy_matches_oracle(dtype):
    mats = [_rm(r, c, 10 + i, dtype) for i, (r, c) in enumerate(ENT_SHAPES)]
    out = woq.ewq_block_entropy(mats)
    h = out["h_mat"].cpu().numpy()
    for i, m in enumerate(mats):
        ref = oracle.matrix_entropy(_np(m))
        assert abs(h[i] - ref) <= 1e-12 * ref, (ENT_SHAPES[i], h[i], ref)


def test_entropy_special_values_and_windows():
    base = _rm(64, 256, 3, std=0.02)
    big = base.float() * 3000.0               # magnitudes beyond the LDS window
    tiny = base.float() * 1e-7                # below the window
    zeros = torch.zeros(16, 64, device=DEV)
    mixed = base.clone()
    mixed[:4] = 0
    mixed[4, :8] = 100.0
    mats = [big.to(torch.bfloat16), tiny.to(torch.bfloat16), zeros.to(torch.bfloat16), mixed,
            torch.full((8, 8), 0.37, device=DEV).to(torch.bfloat16)]
    h = woq.ewq_block_entropy(mats)["h_mat"].cpu().numpy()
    for i, m in enumerate(mats):
        ref = oracle.matrix_entropy(_np(m))
        assert abs(h[i] - ref) <= 1e-12 * max(ref, 1e-300) + 1e-14, (i, h[i], ref)
    assert h[2] == pytest.approx(math.log(16 * 64), rel=1e-14)
    assert h[4] == pytest.approx(math.log(64), rel=1e-14)
    nanm = base.clone()
    nanm[1, 1] = float("nan")
    infm = base.float().clone()
    infm[0, 0] = float("inf")
    h = woq.ewq_block_entropy([nanm, infm])["h_mat"].cpu().numpy()
    assert math.isnan(h[0]) and math.isnan(h[1])


def test_fp32_entropy_running_maximum():
    """fp32 matrices are read once, each thread keeping a running maximum
    that rescales its sums: values rising along every thread's elements (a
    new maximum at each one), falling, spread so widely that most
    exponentials underflow, one outlier far above the rest, all equal, and
    NaN / inf inside one work unit of many-unit matrices."""
    rng = np.random.default_rng(41)
    rise = np.linspace(-30.0, 30.0, 512 * 1024).astype(np.float32).reshape(512, 1024)
    fall = rise[::-1, ::-1].copy()
    wide = ((rng.random((300, 1000)) * 2 - 1) * 3e3).astype(np.float32)
    out1 = (rng.standard_normal((1024, 640)) * 0.02).astype(np.float32)
    out1[700, 33] = 700.0
    out2 = out1.copy()
    out2[5, 5] = 1e4
    flat = np.full((1000, 777), 0.37, dtype=np.float32)
    mats = [torch.from_numpy(a).to(DEV) for a in (rise, fall, wide, out1, out2, flat)]
    h = woq.ewq_block_entropy(mats)["h_mat"].cpu().numpy()
    for i, m in enumerate(mats):
        ref = oracle.matrix_entropy(m.cpu().numpy())
        assert abs(h[i] - ref) <= 1e-12 * ref + 1e-14, (i, h[i], ref)
    assert h[5] == pytest.approx(math.log(1000 * 777), rel=1e-14)
    view = mats[0][:, 256:768]
    assert not view.is_contiguous()
    a = woq.ewq_block_entropy([view])["h_mat"]
    b = woq.ewq_block_entropy([view.contiguous()])["h_mat"]
    assert torch.equal(a.view(torch.int64), b.view(torch.int64))
    bad = torch.from_numpy((rng.standard_normal((2048, 1024)) * 0.02).astype(np.float32)).to(DEV)
    bad2 = bad.clone()
    bad[1500, 3] = float("nan")
    bad2[2047, 1023] = float("-inf")
    bad2[0, 0] = float("inf")
    out = woq.ewq_block_entropy([bad, mats[3], bad2])
    h = out["h_mat"].cpu().numpy()
    assert math.isnan(h[0]) and math.isnan(h[2]) and h[1] == woq.ewq_block_entropy([mats[3]])["h_mat"].item()
    assert out["nonfinite"].item() == 3


def test_block_entropy_tiers_order():
    rng = np.random.default_rng(5)
    mats, bid = [], []
    for b in range(9):
        std = float(rng.uniform(0.01, 0.04))
        for k, (r, c) in enumerate([(64, 128), (32, 128), (96, 64)]):
            mats.append(_rm(r, c, 100 * b + k, std=std))
            bid.append(b)
    out = woq.ewq_block_entropy(mats, bid, 9, x=1.0)
    h_ref = np.array([oracle.matrix_entropy(_np(m)) for m in mats])
    sizes = [m.numel() for m in mats]
    hb_ref = oracle.block_entropy(h_ref, sizes, bid, 9)
    mu, sigma, t, tiers = oracle.ewq_tiers(hb_ref, 1.0)
    np.testing.assert_allclose(out["h_mat"].cpu().numpy(), h_ref, rtol=1e-12)
    np.testing.assert_allclose(out["h_block"].cpu().numpy(), hb_ref, rtol=1e-12)
    np.testing.assert_allclose(out["stats"].cpu().numpy(), [mu, sigma, t], rtol=1e-9, atol=1e-13)
    assert out["tier"].cpu().tolist() == tiers.tolist()
    assert out["order"].cpu().tolist() == oracle.ewq_order(hb_ref).tolist()


@pytest.mark.parametrize("nb", [1000, 4096])
def test_block_statistics_many_blocks(nb):
    """Up to the largest block count (4,096, all kept in LDS by the tier
    kernel), with ties between blocks (every tenth block a copy of the one
    before it): entropies, statistics, tiers and order against the oracle."""
    rng = np.random.default_rng(nb)
    base = [_rm(8, 16, 1000 + i, std=float(rng.uniform(0.005, 0.05))) for i in range(nb)]
    for i in range(10, nb, 10):
        base[i] = base[i - 1].clone()
    out = woq.ewq_block_entropy(base, list(range(nb)), nb, x=0.5)
    hb = out["h_block"].cpu().numpy()
    h_ref = np.array([oracle.matrix_entropy(_np(m)) for m in base])
    np.testing.assert_allclose(hb, h_ref, rtol=1e-12)
    mu, sigma, t, tiers = oracle.ewq_tiers(hb, 0.5)
    np.testing.assert_allclose(out["stats"].cpu().numpy(), [mu, sigma, t], rtol=1e-12)
    got = out["tier"].cpu().numpy()
    near = (np.abs(hb - t) <= 1e-12 * abs(t)) | (np.abs(hb - mu) <= 1e-12 * abs(mu))
    assert np.array_equal(got[~near], tiers[~near])
    assert out["order"].cpu().tolist() == oracle.ewq_order(hb).tolist()


def test_single_block_is_tier_one():
    out = woq.ewq_block_entropy([_rm(8, 16, 1), _rm(8, 16, 2)])
    assert out["tier"].cpu().tolist() == [1]
    assert out["order"].cpu().tolist() == [0]


# ------------------------------------------------------------------ sinkhorn
# wave pass (rows <= 4096 bf16 / 1536 fp32 columns) and workgroup pass, each
# with rows that are and are not a whole number of lane vectors
SINQ_CASES = [((256, 512), torch.float32), ((300, 1024), torch.bfloat16),
              ((64, 2056), torch.bfloat16), ((129, 4104), torch.bfloat16),
              ((1408, 2048), torch.bfloat16), ((2048, 1408), torch.bfloat16), ((5, 8), torch.float32),
              ((96, 14336), torch.bfloat16), ((17, 8192), torch.bfloat16), ((70, 6000), torch.bfloat16),
              ((31, 7000), torch.bfloat16), ((12, 5000), torch.bfloat16),
              ((40, 2048), torch.float32), ((33, 3000), torch.float32)]


@pytest.mark.parametrize("iters", [0, 1, 16])
def test_sinq_matches_oracle(iters):
    mats = [_rm(r, c, 20 + i, dt, frac=0.01, mult=20.0) for i, ((r, c), dt) in enumerate(SINQ_CASES)]
    s, t = woq.sinq_balance(mats, iters)
    for i, m in enumerate(mats):
        s_ref, t_ref = oracle.sinkhorn_std(_np(m), iters)
        np.testing.assert_allclose(s[i].cpu().numpy(), s_ref, rtol=1e-4, err_msg=str(SINQ_CASES[i]))
        np.testing.assert_allclose(t[i].cpu().numpy(), t_ref, rtol=1e-4, err_msg=str(SINQ_CASES[i]))
        # the kernels are far inside the bar
        assert np.max(np.abs(s[i].cpu().numpy() / s_ref - 1)) < 2e-5
        assert np.max(np.abs(t[i].cpu().numpy() / t_ref - 1)) < 2e-5


@pytest.mark.parametrize("shape", [(64, 512), (16, 8192)])
@pytest.mark.parametrize("shared", [False, True])
def test_sinq_plan_of_several_rounds(shared, shape):
    """More same-shape matrices than the GPU holds workgroups at once (600
    of them, wave form and workgroup form: one workgroup sweeps each whole,
    except the last round's matrices, swept in strips of half the height and
    combined by the reduction kernel); the first, middle and last matrices
    against the oracle."""
    mats = [_rm(*shape, 3000 + i, std=0.02 * (1 + i % 5)) for i in range(600)]
    s, t = woq.sinq_balance(mats, 6, shared=shared)
    for i in list(range(0, 600, 37)) + list(range(560, 600)):
        s_ref, t_ref = oracle.sinkhorn_std(_np(mats[i]), 6)
        assert np.max(np.abs(s[i].cpu().numpy() / s_ref - 1)) < 2e-5, i
        assert np.max(np.abs(t[i].cpu().numpy() / t_ref - 1)) < 2e-5, i


def test_sinq_degenerate_lines():
    w = _rm(64, 256, 7).float()
    w[3, :] = 0
    w[5, :] = 0.015625       # constant row (exact bf16)
    w[:, 10] = 0
    wide = _rm(24, 8192, 8).float()
    wide[2, :] = -0.5        # constant rows and a zero column through the workgroup pass
    wide[:, 77] = 0
    wf = _rm(20, 2048, 9, torch.float32)
    wf[4, :] = 0.1           # constant fp32 row (not exact in bf16)
    mats = [w.to(torch.bfloat16), torch.full((16, 32), 0.25, device=DEV).to(torch.bfloat16),
            wide.to(torch.bfloat16), wf]
    s, t = woq.sinq_balance(mats, 6)
    for i, m in enumerate(mats):
        s_ref, t_ref = oracle.sinkhorn_std(_np(m), 6)
        np.testing.assert_allclose(s[i].cpu().numpy(), s_ref, rtol=1e-5)
        np.testing.assert_allclose(t[i].cpu().numpy(), t_ref, rtol=1e-5)
    assert s[0][3].item() == 1.0 and t[0][10].item() == 1.0
    assert torch.all(s[1] == 1) and torch.all(t[1] == 1)
    assert t[2][77].item() == 1.0


@pytest.mark.parametrize("iters", [1, 16])
def test_sinq_rms_variant_matches_oracle(iters):
    """sinq_balance_ex with the root mean square: both passes, both dtypes,
    ragged rows, with a mean added so that centred and uncentred differ."""
    mats = [(_rm(r, c, 40 + i, dt, frac=0.01, mult=20.0).float() + 0.01).to(dt)
            for i, ((r, c), dt) in enumerate(SINQ_CASES)]
    mats[1][7, :] = 0        # a zero row gets scale 1
    s, t = woq.sinq_balance(mats, iters, rms=True)
    for i, m in enumerate(mats):
        s_ref, t_ref = oracle.sinkhorn_std(_np(m), iters, rms=True)
        np.testing.assert_allclose(s[i].cpu().numpy(), s_ref, rtol=1e-4, err_msg=str(SINQ_CASES[i]))
        np.testing.assert_allclose(t[i].cpu().numpy(), t_ref, rtol=1e-4, err_msg=str(SINQ_CASES[i]))
        assert np.max(np.abs(s[i].cpu().numpy() / s_ref - 1)) < 2e-5
        assert np.max(np.abs(t[i].cpu().numpy() / t_ref - 1)) < 2e-5
    assert s[1][7].item() == 1.0
    # the centred result differs (the stds differ by the mean)
    s_c, _ = woq.sinq_balance(mats[:1], iters)
    assert not torch.allclose(s_c[0], s[0], rtol=1e-3)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_sinq_columns_with_large_means(dtype):
    """Columns whose mean is ~100 standard deviations (a common offset; the
    few-row case is in the limits tests): the reduction recomputes them
    around their mean, so the scales stay within the bar instead of losing
    eps * mean^2 / var."""
    w = (_rm(256, 1024, 31, torch.float32) + 2.0).to(dtype)
    w2 = (_rm(64, 14336, 33, torch.float32) - 1.5).to(dtype)     # workgroup pass
    w3 = (_rm(48, 8192, 34, torch.float32) + 0.75).to(dtype)     # two-wave workgroups (bf16)
    s, t = woq.sinq_balance([w, w2, w3], 16)
    for i, m in enumerate((w, w2, w3)):
        s_ref, t_ref = oracle.sinkhorn_std(_np(m), 16)
        np.testing.assert_allclose(s[i].cpu().numpy(), s_ref, rtol=1e-4)
        np.testing.assert_allclose(t[i].cpu().numpy(), t_ref, rtol=1e-4)
        assert np.max(np.abs(t[i].cpu().numpy() / t_ref - 1)) < 2e-5


def test_sinq_deterministic():
    mats = [_rm(512, 2048, 9), _rm(300, 8192, 10), _rm(200, 14336, 11)]
    a = woq.sinq_balance(mats, 16)
    b = woq.sinq_balance(mats, 16)
    for i in range(len(mats)):
        assert torch.equal(a[0][i], b[0][i]) and torch.equal(a[1][i], b[1][i]), i


@pytest.mark.parametrize("iters", [1, 16])
def test_sinq_shared_plan_matches_oracle(iters):
    """WOQ_SINQ_SHARED plans taller strips (half of the GPU): the same scales
    to within the same bar, and within fp32 rounding of the unflagged call."""
    mats = [_rm(r, c, 20 + i, dt, frac=0.01, mult=20.0) for i, ((r, c), dt) in enumerate(SINQ_CASES)]
    s, t = woq.sinq_balance(mats, iters, shared=True)
    s0, t0 = woq.sinq_balance(mats, iters)
    for i, m in enumerate(mats):
        s_ref, t_ref = oracle.sinkhorn_std(_np(m), iters)
        np.testing.assert_allclose(s[i].cpu().numpy(), s_ref, rtol=1e-4, err_msg=str(SINQ_CASES[i]))
        np.testing.assert_allclose(t[i].cpu().numpy(), t_ref, rtol=1e-4, err_msg=str(SINQ_CASES[i]))
        np.testing.assert_allclose(s[i].cpu().numpy(), s0[i].cpu().numpy(), rtol=2e-5)
        np.testing.assert_allclose(t[i].cpu().numpy(), t0[i].cpu().numpy(), rtol=2e-5)


def test_sinq_concurrent_calls_on_two_streams():
    """The pipeline's split: wave-form matrices on one stream, wider ones with
    WOQ_SINQ_SHARED on another, each with its own workspace.  Every result
    equals the same call made alone, bit for bit, on every repetition."""
    narrow = [_rm(1024, 4096, 31), _rm(4096, 4096, 32), _rm(300, 1024, 33)]
    wide = [_rm(4096, 14336, 34), _rm(96, 14336, 35)]
    ref_n = woq.sinq_balance(narrow, 16)
    ref_w = woq.sinq_balance(wide, 16, shared=True)
    from weight_only_quantization_softmax_amd import _lib
    ws_n = torch.empty(woq.workspace_size(_lib.OP_SINQ, narrow), dtype=torch.uint8, device=DEV)
    ws_w = torch.empty(woq.workspace_size(_lib.OP_SINQ, wide), dtype=torch.uint8, device=DEV)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    for rep in range(3):
        sn = [torch.empty_like(x) for x in ref_n[0]]
        tn = [torch.empty_like(x) for x in ref_n[1]]
        sw = [torch.empty_like(x) for x in ref_w[0]]
        tw = [torch.empty_like(x) for x in ref_w[1]]
        side.wait_stream(main)
        woq.sinq_balance(narrow, 16, row_scale=sn, col_scale=tn, ws=ws_n, stream=main)
        woq.sinq_balance(wide, 16, shared=True, row_scale=sw, col_scale=tw, ws=ws_w, stream=side)
        main.wait_stream(side)
        torch.cuda.synchronize()
        for a, b in zip(sn + tn + sw + tw, ref_n[0] + ref_n[1] + ref_w[0] + ref_w[1]):
            assert torch.equal(a, b), rep


# ------------------------------------------------------------------ quant
QUANT_CASES = [  # (rows, cols, bits, group, dtype)
    (16, 256, 4, 64, torch.bfloat16), (7, 96, 4, 32, torch.bfloat16),
    (33, 384, 3, 128, torch.bfloat16), (9, 512, 2, 8, torch.bfloat16),
    (12, 1024, 8, 512, torch.bfloat16), (5, 4096, 8, 0, torch.bfloat16),
    (3, 14336, 8, 0, torch.bfloat16), (20, 2048, 4, 1024, torch.bfloat16),
    (256, 512, 4, 64, torch.float32), (11, 1408, 4, 64, torch.bfloat16),
    (4, 3072, 3, 0, torch.float32), (2, 64, 8, 16, torch.float32),
    # several 2048-column tiles with a ragged last one; groups of 600 (one
    # wave, lanes with no vector); two 8192-column groups per row (workgroup)
    (13, 2560, 4, 64, torch.bfloat16), (9, 6144, 4, 128, torch.bfloat16),
    (10, 1800, 4, 600, torch.bfloat16), (4, 16384, 4, 8192, torch.bfloat16),
    # 3-bit rows whose codes start at odd byte offsets, ragged tiles
    (7, 136, 3, 8, torch.bfloat16), (5, 2600, 3, 8, torch.float32), (6, 4104, 3, 8, torch.bfloat16),
]


def _check_quant(m, s, t, bits, group, codes, scales, zeros):
    w = _np(m)
    g = group if group else w.shape[1]
    sn = None if s is None else s.cpu().numpy()
    tn = None if t is None else t.cpu().numpy()
    q_ref, d_ref, z_ref = oracle.quantize_groupwise_f32(w, sn, tn, bits, g)
    packed_ref = oracle.pack_codes(q_ref, bits)
    d = scales.cpu().numpy()
    assert np.array_equal(d.view(np.uint32), d_ref.view(np.uint32))
    assert np.array_equal(zeros.cpu().numpy(), z_ref)
    assert np.array_equal(codes.cpu().numpy(), packed_ref)


@pytest.mark.parametrize("with_scales", [False, True])
def test_quant_bit_exact(with_scales):
    counts = []
    for i, (r, c, bits, group, dt) in enumerate(QUANT_CASES):
        m = _rm(r, c, 40 + i, dt, frac=0.01, mult=20.0)
        s = t = None
        if with_scales:
            ss, tt = woq.sinq_balance([m], 3)
            s, t = ss[0], tt[0]
        codes, scales, zeros = woq.quant_pack_groupwise(
            [m], bits, group, row_scale=None if s is None else [s],
            col_scale=None if t is None else [t])
        _check_quant(m, s, t, bits, group, codes[0], scales[0], zeros[0])
        g = group if group else c
        q = oracle.unpack_codes(codes[0].cpu().numpy(), bits, c)
        counts.append(_codes.affine(_np(m), None if s is None else s.cpu().numpy(),
                                    None if t is None else t.cpu().numpy(), bits, g, q))
    _codes.within_budget(counts)


def test_quant_exact_half_way_points():
    """bf16 weights on a coarse lattice, symmetric groups and per-row groups
    whose largest and smallest weights cancel: many ratios are exact half-way
    points.  The kernels decide every one as the fp64 definition does (the
    zero-point and near-half ratios by a correctly rounded division): no
    difference at all, on all three quantise kernels."""
    g = torch.Generator(device="cpu").manual_seed(5)
    for rows, cols, bits, group in [(64, 1024, 4, 64), (48, 4096, 8, 0), (16, 14336, 8, 0),
                                    (32, 1800, 8, 600), (64, 512, 3, 128), (64, 256, 2, 32)]:
        x = torch.randint(-24, 25, (rows, cols), generator=g).float() * 2.0 ** -7
        gg = group if group else cols
        x[:, gg - 1] = -x[:, :gg - 1].abs().amax(dim=1)     # hi = -lo in the first group
        x[0, :gg] = torch.linspace(-1, 1, gg)
        m = x.to(torch.bfloat16).to(DEV)
        codes, scales, zeros = woq.quant_pack_groupwise([m], bits, group)
        _check_quant(m, None, None, bits, group, codes[0], scales[0], zeros[0])
        q = oracle.unpack_codes(codes[0].cpu().numpy(), bits, cols)
        w = _np(m)
        assert np.array_equal(q, oracle.quantize_groupwise_f64(w, None, None, bits, gg)[0]), (rows, cols)
        assert oracle.near_tie_mask(w, None, None, bits, gg, 1e-12).any()


def test_quant_batched_mixed_dtypes_and_edge_groups():
    mats = [_rm(16, 256, 1), _rm(8, 512, 2, torch.float32), _rm(4, 64, 3)]
    mats.append(torch.zeros(2, 128, device=DEV, dtype=torch.bfloat16))       # delta = 0 groups
    c = torch.full((2, 128), 0.5, device=DEV)
    c[1, 64:] = -0.25
    mats.append(c.to(torch.bfloat16))                                         # one-signed groups
    codes, scales, zeros = woq.quant_pack_groupwise(mats, 4, 64)
    for i, m in enumerate(mats):
        _check_quant(m, None, None, 4, 64, codes[i], scales[i], zeros[i])
    assert torch.all(scales[3] == 0) and torch.all(codes[3] == 0)


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("bits,group,rows,cols", [(4, 64, 24, 1024), (3, 128, 24, 1024),
                                                  (8, 0, 24, 1024), (2, 32, 24, 1024),
                                                  (4, 64, 13, 2560), (3, 128, 9, 6144)])
def test_dequant_matches_oracle(bits, group, rows, cols):
    m = _rm(rows, cols, 61)
    ss, tt = woq.sinq_balance([m], 2)
    codes, scales, zeros = woq.quant_pack_groupwise([m], bits, group, row_scale=ss, col_scale=tt)
    g = group if group else cols
    q_ref = oracle.unpack_codes(codes[0].cpu().numpy(), bits, cols)
    ref = oracle.dequantize_f32(q_ref, scales[0].cpu().numpy(), zeros[0].cpu().numpy(),
                                ss[0].cpu().numpy(), tt[0].cpu().numpy(), g)
    out32 = woq.dequant_unpack([(rows, cols)], codes, scales, bits, group, zeros=zeros,
                               row_scale=ss, col_scale=tt)[0]
    assert np.array_equal(out32.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    out16 = woq.dequant_unpack([(rows, cols)], codes, scales, bits, group, zeros=zeros,
                               row_scale=ss, col_scale=tt, out_dtype=torch.bfloat16)[0]
    assert torch.equal(out16.cpu(), torch.from_numpy(ref).to(torch.bfloat16))
    # error bound: |W - W'| <= s t delta / 2 (plus fp32 rounding)
    w = _np(m).astype(np.float64)
    bound = np.outer(ss[0].cpu().numpy(), tt[0].cpu().numpy()) * np.repeat(scales[0].cpu().numpy(), g, 1) / 2
    assert np.all(np.abs(w - ref) <= bound * (1 + 1e-4) + 1e-12)


# ------------------------------------------------------------------ ternary
# rows of up to 4096 columns take one wave per row (8-column vectors per
# lane: 1, 2, 4, 8), wider rows one workgroup per row; row counts off the
# 16-row unit
@pytest.mark.parametrize("shape,dtype", [((64, 2048), torch.bfloat16), ((33, 1408), torch.bfloat16),
                                         ((7, 4096), torch.float32), ((3, 16), torch.bfloat16),
                                         ((17, 512), torch.bfloat16), ((100, 1024), torch.float32),
                                         ((5, 4104), torch.bfloat16), ((40, 6144), torch.float32)])
def test_ternary_matches_oracle(shape, dtype):
    m = _rm(*shape, 71, dtype)
    m[0] = 0  # beta = 0 row
    codes, beta = woq.ternary_pack([m])
    q_ref, b_ref = oracle.ternary_quantize(_np(m))
    assert np.array_equal(beta[0].cpu().numpy().view(np.uint32), b_ref.view(np.uint32))
    packed = oracle.pack_codes((q_ref + 1).astype(np.uint8), 2)
    assert np.array_equal(codes[0].cpu().numpy(), packed)
    q_gpu = oracle.unpack_codes(codes[0].cpu().numpy(), 2, shape[1]).astype(np.int8) - 1
    n, tot = _codes.ternary(_np(m), q_gpu)
    assert n <= max(1, 1e-5 * tot)
    deq = woq.dequant_unpack([shape], codes, [beta[0]], 2, 0)[0]
    assert np.array_equal(deq.cpu().numpy(), oracle.ternary_dequantize(q_ref, b_ref))


def test_ternary_batch_of_launch_sets_equals_single_calls():
    """One call over matrices of every launch set (both dtypes, wave and
    workgroup forms, interleaved) gives each matrix what a call on it alone
    gives."""
    shapes = [(33, 1408, torch.bfloat16), (9, 8192, torch.bfloat16), (48, 512, torch.float32),
              (16, 2048, torch.bfloat16), (2, 4104, torch.float32), (70, 1024, torch.bfloat16),
              (1, 8, torch.float32)]
    mats = [_rm(r, c, 80 + i, dt) for i, (r, c, dt) in enumerate(shapes)]
    codes, beta = woq.ternary_pack(mats)
    for i, m in enumerate(mats):
        c1, b1 = woq.ternary_pack([m])
        assert torch.equal(codes[i], c1[0]), shapes[i]
        assert torch.equal(beta[i].view(torch.int32), b1[0].view(torch.int32)), shapes[i]


# ------------------------------------------------------------------ end to end (single fp32 workload)
def test_single_matrix_workload_end_to_end():
    wl, specs, ws = woqdata.generate("single")
    w = ws[0].to(DEV)
    h = woq.ewq_block_entropy([w])["h_mat"].item()
    assert abs(h - oracle.matrix_entropy(w.cpu().numpy())) <= 1e-12 * h
    s, t = woq.sinq_balance([w], wl.iters)
    s_ref, t_ref = oracle.sinkhorn_std(w.cpu().numpy(), wl.iters)
    np.testing.assert_allclose(s[0].cpu().numpy(), s_ref, rtol=1e-4)
    np.testing.assert_allclose(t[0].cpu().numpy(), t_ref, rtol=1e-4)
    codes, scales, zeros = woq.quant_pack_groupwise([w], wl.bits, wl.group, row_scale=s, col_scale=t)
    _check_quant(w, s[0], t[0], wl.bits, wl.group, codes[0], scales[0], zeros[0])
    # the fp64 definition fed with the same scales: only near ties may differ
    sg, tg = s[0].cpu().numpy(), t[0].cpu().numpy()
    q_gpu = oracle.unpack_codes(codes[0].cpu().numpy(), wl.bits, 512)
    _codes.within_budget([_codes.affine(w.cpu().numpy(), sg, tg, wl.bits, wl.group, q_gpu)])
    # fully independent fp64 path (its own scales): codes move by at most
    # one, on at most 1e-4 of the 131,072 (13 codes; the 1e-5 bar is
    # checked on the full-size workloads, where it is meaningful)
    n, tot = _codes.end_to_end(w.cpu().numpy(), s_ref, t_ref, wl.bits, wl.group, q_gpu)
    assert n <= 1e-4 * tot
