"""Full-size parity of the tier pipeline (QuantPass) on the workloads' own
shapes, in the launch configuration the benchmark times.

The CPU oracle checks sampled outputs one matrix (or one row set) at a time;
outputs too large for it are checked through properties that hold at any
size: after the final column step every column of W / (s t^T) has std 1 and
the row stds agree with each other, and codes are row-local given (s, t), so
sampled rows are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import woqdata
from weight_only_quantization_softmax_amd.pipeline import QuantPass

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return t.float().cpu().numpy()


def _pass(wl, specs, mats, tiered=None):
    blocks = sorted({m.block for m in specs})
    remap = {b: i for i, b in enumerate(blocks)}
    qp = QuantPass(mats, [remap[m.block] for m in specs], len(blocks), iters=wl.iters,
                   bits=wl.bits, group=wl.group, x=wl.x,
                   tiered=wl.tiered if tiered is None else tiered,
                   actions=(wl.low_tier, wl.mid_tier, wl.high_tier))
    tiers = qp.run()
    torch.cuda.synchronize()
    return qp, tiers


def _check_sinq_matrix(w, out, iters, bits, group):
    s_ref, t_ref = oracle.sinkhorn_std(w, iters)
    s, t = out["s"].cpu().numpy(), out["t"].cpu().numpy()
    np.testing.assert_allclose(s, s_ref, rtol=1e-4)
    np.testing.assert_allclose(t, t_ref, rtol=1e-4)
    q, d, z = oracle.quantize_groupwise_f32(w, s, t, bits, group)
    assert np.array_equal(out["codes"].cpu().numpy(), oracle.pack_codes(q, bits))
    assert np.array_equal(out["scales"].cpu().numpy().view(np.uint32), d.view(np.uint32))
    assert np.array_equal(out["zeros"].cpu().numpy(), z)


def _check_balance_properties(m, out, row_spread):
    """Column stds of W / (s t^T) equal 1; row stds agree (fp64 on the device)."""
    b = m.double() / (out["s"].double()[:, None] * out["t"].double()[None, :])
    col = b.std(dim=0, unbiased=False)
    row = b.std(dim=1, unbiased=False)
    assert torch.max(torch.abs(col - 1)).item() < 1e-4
    assert (row.max() / row.min() - 1).item() < row_spread
    del b


def _check_rows(m, out, bits, group, rows):
    w = _np(m[rows])
    s = out["s"].cpu().numpy()[rows]
    t = out["t"].cpu().numpy()
    q, d, z = oracle.quantize_groupwise_f32(w, s, t, bits, group)
    rb = m.shape[1] * bits // 8
    codes = out["codes"].cpu().numpy().reshape(m.shape[0], rb)[rows]
    assert np.array_equal(codes, oracle.pack_codes(q, bits))
    assert np.array_equal(out["scales"].cpu().numpy()[rows].view(np.uint32), d.view(np.uint32))
    assert np.array_equal(out["zeros"].cpu().numpy()[rows], z)


def test_block_workload_full_size():
    """One Llama-3.1-8B block: entropy of all 7 matrices, Sinkhorn K=16 + int4 g64."""
    wl, specs, mats = woqdata.generate("block", device=DEV)
    qp, tiers = _pass(wl, specs, mats)
    h = qp.h_mat.cpu().numpy()
    for i, m in enumerate(mats):
        np.testing.assert_allclose(h[i], oracle.matrix_entropy(_np(m)), rtol=1e-10, err_msg=specs[i].name)
    hb = oracle.block_entropy(h, [m.numel() for m in mats], [0] * 7, 1)
    np.testing.assert_allclose(qp.h_block.cpu().numpy(), hb, rtol=1e-12)
    for i in (1, 2):   # k and v through the oracle in full
        _check_sinq_matrix(_np(mats[i]), qp.outputs[i], wl.iters, wl.bits, wl.group)
    rng = np.random.default_rng(0)
    for i in (4, 6):   # gate (wave pass) and down (workgroup pass): properties + sampled rows
        _check_balance_properties(mats[i], qp.outputs[i], 1e-4)
        rows = np.sort(rng.choice(mats[i].shape[0], 48, replace=False))
        _check_rows(mats[i], qp.outputs[i], wl.bits, wl.group, rows)


def test_stack8b_full_configuration():
    """The benchmark's configuration: 32 blocks, tiers at X = 1, mixed calls."""
    wl, specs, mats = woqdata.generate("stack8b", device=DEV)
    qp, tiers = _pass(wl, specs, mats)
    h = qp.h_mat.cpu().numpy()
    bid = [m.block for m in specs]
    # block statistics and tiers from the device entropies (stage isolation)
    hb = oracle.block_entropy(h, [m.numel() for m in mats], bid, wl.n_blocks)
    np.testing.assert_allclose(qp.h_block.cpu().numpy(), hb, rtol=1e-12)
    mu, sigma, t_thr, tier_ref = oracle.ewq_tiers(hb)
    assert qp.tier.cpu().tolist() == tier_ref.tolist()
    assert tiers == tier_ref.tolist()
    rng = np.random.default_rng(1)
    acts = qp.action_of_block(tiers)
    seen = set()
    for i in rng.permutation(len(mats)):
        a = acts[bid[i]]
        if a in seen or specs[i].name.split(".")[-1] not in ("k", "v"):
            continue
        seen.add(a)
        w = _np(mats[i])
        np.testing.assert_allclose(h[i], oracle.matrix_entropy(w), rtol=1e-10)
        out = qp.outputs[i]
        if a == "sinq":
            _check_sinq_matrix(w, out, wl.iters, wl.bits, wl.group)
        elif a == "int8row":
            q, d, z = oracle.quantize_groupwise_f32(w, None, None, 8, w.shape[1])
            assert np.array_equal(out["codes"].cpu().numpy(), oracle.pack_codes(q, 8))
            assert np.array_equal(out["scales"].cpu().numpy().reshape(-1).view(np.uint32),
                                  d.reshape(-1).view(np.uint32))
        else:
            assert a == "keep" and set(out) == {"action"}
    assert seen == {"sinq", "int8row", "keep"}


def test_stack70b_block_int3():
    """One 70B-shaped block: K = 24, int3 g128, 8192- and 28672-column rows."""
    wl, specs, mats = woqdata.generate("stack70b", device=DEV, blocks=[0])
    qp, tiers = _pass(wl, specs, mats, tiered=False)
    h = qp.h_mat.cpu().numpy()
    for i in (1, 2):   # k, v: 1024 x 8192 through the oracle in full
        w = _np(mats[i])
        np.testing.assert_allclose(h[i], oracle.matrix_entropy(w), rtol=1e-10)
        _check_sinq_matrix(w, qp.outputs[i], wl.iters, wl.bits, wl.group)
    rng = np.random.default_rng(2)
    for i in (0, 6):   # q (8192 columns) and down (28672 columns, 512-thread workgroups)
        _check_balance_properties(mats[i], qp.outputs[i], 1e-4)
        rows = np.sort(rng.choice(mats[i].shape[0], 32, replace=False))
        _check_rows(mats[i], qp.outputs[i], wl.bits, wl.group, rows)


def test_moe_layers_tiered():
    """Four MoE layers (784 matrices): tiers over layers, ternary lowest tier."""
    wl, specs, mats = woqdata.generate("moe", device=DEV, blocks=[0, 1, 2, 3])
    qp, tiers = _pass(wl, specs, mats)
    h = qp.h_mat.cpu().numpy()
    bid = [m.block for m in specs]
    hb = oracle.block_entropy(h, [m.numel() for m in mats], bid, 4)
    assert qp.tier.cpu().tolist() == oracle.ewq_tiers(hb)[3].tolist()
    acts = qp.action_of_block(tiers)
    rng = np.random.default_rng(3)
    sample = list(range(4)) + [int(i) for i in rng.choice(len(mats), 12, replace=False)]
    for i in sample:
        w = _np(mats[i])
        np.testing.assert_allclose(h[i], oracle.matrix_entropy(w), rtol=1e-10, err_msg=specs[i].name)
        out = qp.outputs[i]
        a = acts[bid[i]]
        if a == "ternary":
            q, beta = oracle.ternary_quantize(w)
            assert np.array_equal(out["beta"].cpu().numpy(), beta)
            assert np.array_equal(out["codes"].cpu().numpy(),
                                  oracle.pack_codes((q + 1).astype(np.uint8), 2))
        else:
            assert a == "sinq"
            _check_sinq_matrix(w, out, wl.iters, wl.bits, wl.group)


def test_quality_report_rows():
    """The data-free report: one row per (scheme, K) plus ternary, all finite;
    at every K the 4-bit g64 error is below the 3-bit g128 error on both
    grids, and the largest error is within the per-element rounding bound
    (max(s t delta) / 2 affine, max(s t a) G / 2 for the code book)."""
    from weight_only_quantization_softmax_amd import quality
    w = woqdata.random_matrix(256, 1024, 77, device=DEV)
    rows = quality.matrix_report(w)
    nk = sum(1 for k in quality.ITERS if k)
    assert len(rows) == len(quality.SCHEMES) * (1 + nk * len(quality.STDS)) + 1
    assert all(np.isfinite(r["rel_fro"]) and np.isfinite(r["max_abs"]) for r in rows)
    by = {(r["scheme"], r["iters"], r["std"]): r for r in rows}
    import weight_only_quantization_softmax_amd as woq
    for k in quality.ITERS:
        for std in (quality.STDS if k else ("none",)):
            assert by[("int4 g64", k, std)]["rel_fro"] < by[("int3 g128", k, std)]["rel_fro"]
            s, t = woq.sinq_balance([w], k, rms=(std == "rms"))
            _, scales, _ = woq.quant_pack_groupwise([w], 4, 64, row_scale=s, col_scale=t)
            bound = (s[0][:, None].double() * t[0][None, :].double()
                     * scales[0].double().repeat_interleave(64, dim=1)).max().item() / 2
            assert by[("int4 g64", k, std)]["max_abs"] <= bound * (1 + 1e-5)
            # the normal-quantile book: its error is within the bound that its
            # widest level gap gives, s t a G / 2
            assert by[("nf4 g64", k, std)]["rel_fro"] < by[("nf3 g128", k, std)]["rel_fro"]
            _, a = woq.quant_pack_codebook([w], 4, 64, row_scale=s, col_scale=t)
            lv = woq.codebook_normal(4)
            gap = max(b - a_ for a_, b in zip(lv, lv[1:]))
            bound = (s[0][:, None].double() * t[0][None, :].double()
                     * a[0].double().repeat_interleave(64, dim=1)).max().item() * gap / 2
            assert by[("nf4 g64", k, std)]["max_abs"] <= bound * (1 + 1e-5)
    assert 0 < by[("ternary", 0, "none")]["rel_fro"] < 1


def test_budgeted_placement_moe_layers():
    """EWQ step 3 on four MoE layers: a budget below the tiers' storage
    demotes the lowest-entropy layers first; the pass then runs the moved
    actions and every output is present and within the budget."""
    import weight_only_quantization_softmax_amd as woq
    wl, specs, mats = woqdata.generate("moe", device=DEV, blocks=[0, 1, 2, 3])
    bid = [m.block for m in specs]
    probe = QuantPass(mats, bid, 4, iters=wl.iters, bits=wl.bits, group=wl.group,
                      actions=(wl.low_tier, wl.mid_tier, wl.high_tier))
    tiers0 = probe.run()
    torch.cuda.synchronize()
    lb = probe.level_bytes()
    from weight_only_quantization_softmax_amd.pipeline import ACTIONS
    level0 = [ACTIONS.index(a) for a in probe.action_of_block(tiers0)]
    start = sum(lb[b][level0[b]] for b in range(4))
    hb = probe.h_block.cpu().tolist()
    for budget in (start - 1, (start + sum(r[0] for r in lb)) // 2, start + 10**9):
        qp = QuantPass(mats, bid, 4, iters=wl.iters, bits=wl.bits, group=wl.group,
                       actions=(wl.low_tier, wl.mid_tier, wl.high_tier), budget_bytes=budget)
        qp.run()
        torch.cuda.synchronize()
        ref_lev, ref_total, ref_fits = oracle.ewq_budget(hb, lb, level0, budget)
        assert [ACTIONS.index(a) for a in qp.last_actions] == ref_lev.tolist()
        assert qp.last_budget == (ref_total, ref_fits) and ref_fits
        # storage actually produced equals the planned total
        produced = 0
        for i, m in enumerate(mats):
            out = qp.outputs[i]
            assert out["action"] == qp.last_actions[bid[i]]
            produced += qp.action_bytes(out["action"], m)
        assert produced == ref_total <= budget
    assert woq.ewq_budget_levels(hb, lb, level0, 0)[2] is False


def test_kept_blocks_lossless_code():
    """The pass's kept blocks stored with the lossless exponent code: every
    word decodes exactly and the kept storage is about 11 bits per weight."""
    import weight_only_quantization_softmax_amd as woq
    wl, specs, mats = woqdata.generate("stack8b", device=DEV, blocks=[0, 1, 2, 3])
    qp, tiers = _pass(wl, specs, mats)
    stored = qp.compress_kept()
    torch.cuda.synchronize()
    kept = [i for i, o in qp.outputs.items() if o["action"] == "keep"]
    assert kept and all("df11" in qp.outputs[i] for i in kept)
    outs = woq.df11_decode([qp.outputs[i]["df11"] for i in kept])
    for i, o in zip(kept, outs):
        assert torch.equal(o.view(torch.int16), mats[i].view(torch.int16))
    n = sum(mats[i].numel() for i in kept)
    assert 10.3 < 8 * stored / n < 11.3
