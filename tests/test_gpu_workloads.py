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
from tests import _codes, _par
from weight_only_quantization_softmax_amd.pipeline import QuantPass

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _np(t):
    return _par.host_f32(t)


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


def _release():
    """Return the cached device memory of a finished full-size test (its
    tensors already dropped) so the next configuration fits."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _check_sinq_matrix(w, out, iters, bits, group):
    """Scales against the oracle (1e-4, internal 2e-5); codes, deltas and
    zero-points bit-exact against the fp32 decision sequence fed the GPU's
    scales; codes against the fp64 definition (GPU scales: near ties only)
    and end to end (the oracle's scales).  Returns the two (mismatches,
    elements) counts."""
    s_ref, t_ref = oracle.sinkhorn_std(w, iters)
    s, t = out["s"].cpu().numpy(), out["t"].cpu().numpy()
    np.testing.assert_allclose(s, s_ref, rtol=1e-4)
    np.testing.assert_allclose(t, t_ref, rtol=1e-4)
    assert np.max(np.abs(s / s_ref - 1)) < 2e-5 and np.max(np.abs(t / t_ref - 1)) < 2e-5
    q, d, z = oracle.quantize_groupwise_f32(w, s, t, bits, group)
    codes = out["codes"].cpu().numpy()
    assert np.array_equal(codes, oracle.pack_codes(q, bits))
    assert np.array_equal(out["scales"].cpu().numpy().view(np.uint32), d.view(np.uint32))
    assert np.array_equal(out["zeros"].cpu().numpy(), z)
    q_gpu = oracle.unpack_codes(codes.reshape(w.shape[0], -1), bits, w.shape[1])
    return (_codes.affine(w, s, t, bits, group, q_gpu),
            _codes.end_to_end(w, s_ref, t_ref, bits, group, q_gpu))


def _check_int8_rows(w, out):
    """int8 per row, no balancing: bit-exact against the fp32 sequence and
    against the fp64 definition (exact half-way points included)."""
    q, d, z = oracle.quantize_groupwise_f32(w, None, None, 8, w.shape[1])
    codes = out["codes"].cpu().numpy().reshape(w.shape)
    assert np.array_equal(codes, oracle.pack_codes(q, 8))
    assert np.array_equal(out["scales"].cpu().numpy().reshape(-1).view(np.uint32),
                          d.reshape(-1).view(np.uint32))
    return _codes.affine(w, None, None, 8, w.shape[1], codes)


def _check_ternary(w, out):
    q, beta = oracle.ternary_quantize(w)
    assert np.array_equal(out["beta"].cpu().numpy(), beta)
    codes = out["codes"].cpu().numpy()
    assert np.array_equal(codes, oracle.pack_codes((q + 1).astype(np.uint8), 2))
    q_gpu = oracle.unpack_codes(codes.reshape(w.shape[0], -1), 2, w.shape[1]).astype(np.int8) - 1
    return _codes.ternary(w, q_gpu)


def _check_balance_properties(m, out, row_spread):
    """Column stds of W / (s t^T) equal 1; row stds agree (fp64 on the device)."""
    b = m.double() / (out["s"].double()[:, None] * out["t"].double()[None, :])
    col = b.std(dim=0, unbiased=False)
    row = b.std(dim=1, unbiased=False)
    assert torch.max(torch.abs(col - 1)).item() < 1e-4
    assert (row.max() / row.min() - 1).item() < row_spread
    del b


def _check_rows(m, out, bits, group, rows):
    """Codes are row-local given (s, t): sampled rows bit-exact against the
    fp32 sequence, and against the fp64 definition; returns the count."""
    w = _np(m[rows])
    s = out["s"].cpu().numpy()[rows]
    t = out["t"].cpu().numpy()
    q, d, z = oracle.quantize_groupwise_f32(w, s, t, bits, group)
    rb = m.shape[1] * bits // 8
    codes = out["codes"].cpu().numpy().reshape(m.shape[0], rb)[rows]
    assert np.array_equal(codes, oracle.pack_codes(q, bits))
    assert np.array_equal(out["scales"].cpu().numpy()[rows].view(np.uint32), d.view(np.uint32))
    assert np.array_equal(out["zeros"].cpu().numpy()[rows], z)
    return _codes.affine(w, s, t, bits, group, oracle.unpack_codes(codes, bits, m.shape[1]))


def _oracle_entropies(mats, idx=None):
    idx = range(len(mats)) if idx is None else idx
    return dict(zip(idx, _par.pmap(lambda i: oracle.matrix_entropy(_np(mats[i])), idx)))


def _tier_parity(h_ref, sizes, bid, n_blocks, tier_gpu, eps=1e-7):
    """Tiers from the oracle's own entropies equal the GPU's, except for
    blocks within eps of T or mu (the 1e-5 entropy bar cannot order those).
    Returns the number of such blocks."""
    hb = oracle.block_entropy(h_ref, sizes, bid, n_blocks)
    mu, sigma, t, tiers = oracle.ewq_tiers(hb)
    near = (np.abs(hb - t) < eps) | (np.abs(hb - mu) < eps)
    tg = np.asarray(tier_gpu)
    assert np.array_equal(tiers[~near], tg[~near]), (tiers.tolist(), tg.tolist())
    return int(near.sum())


def test_block_workload_full_size():
    """One Llama-3.1-8B block: entropy of all 7 matrices, Sinkhorn K=16 + int4 g64."""
    wl, specs, mats = woqdata.generate("block", device=DEV)
    qp, tiers = _pass(wl, specs, mats)
    h = qp.h_mat.cpu().numpy()
    h_ref = _oracle_entropies(mats)
    for i in range(len(mats)):
        np.testing.assert_allclose(h[i], h_ref[i], rtol=1e-10, err_msg=specs[i].name)
    hb = oracle.block_entropy(h, [m.numel() for m in mats], [0] * 7, 1)
    np.testing.assert_allclose(qp.h_block.cpu().numpy(), hb, rtol=1e-12)
    iso, e2e = [], []
    res = _par.pmap(lambda i: _check_sinq_matrix(_np(mats[i]), qp.outputs[i], wl.iters, wl.bits,
                                                 wl.group), (1, 2))   # k and v in full
    for a, b in res:
        iso.append(a)
        e2e.append(b)
    rng = np.random.default_rng(0)
    for i in (0, 4, 6):   # q, gate (wave pass) and down (workgroup pass): properties + sampled rows
        _check_balance_properties(mats[i], qp.outputs[i], 1e-4)
        rows = np.sort(rng.choice(mats[i].shape[0], 64, replace=False))
        iso.append(_check_rows(mats[i], qp.outputs[i], wl.bits, wl.group, rows))
    _codes.within_budget(iso)
    _codes.within_budget(e2e)


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_stack8b_full_configuration():
    """The benchmark's configuration: 32 blocks, tiers at X = 1, mixed calls.
    Tiers from the oracle's entropies of all 224 matrices; every action
    checked on sampled matrices of every block that takes it."""
    wl, specs, mats = woqdata.generate("stack8b", device=DEV)
    qp, tiers = _pass(wl, specs, mats)
    h = qp.h_mat.cpu().numpy()
    bid = [m.block for m in specs]
    sizes = [m.numel() for m in mats]
    print(f"[stack8b] tiers {tiers}", flush=True)
    hb = oracle.block_entropy(h, sizes, bid, wl.n_blocks)
    np.testing.assert_allclose(qp.h_block.cpu().numpy(), hb, rtol=1e-12)
    assert tiers == qp.tier.cpu().tolist() == oracle.ewq_tiers(hb)[3].tolist()
    h_ref = _oracle_entropies(mats)
    print("[stack8b] oracle entropies done", flush=True)
    ent_err = max(abs(h[i] / h_ref[i] - 1) for i in range(len(mats)))
    assert ent_err < 1e-10, ent_err
    near = _tier_parity(np.array([h_ref[i] for i in range(len(mats))]), sizes, bid, wl.n_blocks,
                        tiers)
    print(f"[stack8b] max entropy rel err {ent_err:.2e}; blocks within 1e-7 of T or mu: {near}",
          flush=True)
    acts = qp.action_of_block(tiers)
    assert set(acts) == {"sinq", "int8row", "keep"}
    kv = [i for i, sp in enumerate(specs) if sp.name.split(".")[-1] in ("k", "v")]
    sinq_kv = [i for i in kv if acts[bid[i]] == "sinq"]
    int8_kv = [i for i in kv if acts[bid[i]] == "int8row"]
    res = _par.pmap(lambda i: _check_sinq_matrix(_np(mats[i]), qp.outputs[i], wl.iters, wl.bits,
                                                 wl.group), sinq_kv)
    iso = [a for a, _ in res]
    e2e = [b for _, b in res]
    iso += _par.pmap(lambda i: _check_int8_rows(_np(mats[i]), qp.outputs[i]), int8_kv)
    print(f"[stack8b] k/v of {len(sinq_kv) // 2} Sinkhorn and {len(int8_kv) // 2} int8 blocks done",
          flush=True)
    rng = np.random.default_rng(1)
    for b in sorted({bid[i] for i in sinq_kv}):
        for name in ("q", "gate", "down"):
            i = specs.index(next(sp for sp in specs if sp.name == f"b{b}.{name}"))
            rows = np.sort(rng.choice(mats[i].shape[0], 16, replace=False))
            iso.append(_check_rows(mats[i], qp.outputs[i], wl.bits, wl.group, rows))
    for i, sp in enumerate(specs):
        if acts[bid[i]] == "keep":
            assert set(qp.outputs[i]) == {"action"}
    bad, tot = _codes.within_budget(iso)
    print(f"[stack8b] codes vs the fp64 definition: {bad} near-tie differences in {tot}", flush=True)
    bad, tot = _codes.within_budget(e2e)
    print(f"[stack8b] codes end to end: {bad} in {tot}", flush=True)
    del qp, mats
    _release()


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_stack70b_full_configuration():
    """All 80 70B-shaped blocks (137 GB resident): entropies of all 560
    matrices on the GPU, the oracle on blocks 0, 40 and 79; every matrix
    through K = 24 + int3 g128; k and v of those blocks through the oracle
    in full, q and down on sampled rows and the balance properties."""
    wl, specs, mats = woqdata.generate("stack70b", device=DEV)
    torch.cuda.synchronize()
    print(f"[stack70b] {len(mats)} matrices generated", flush=True)
    qp, tiers = _pass(wl, specs, mats, tiered=False)
    h = qp.h_mat.cpu().numpy()
    bid = [m.block for m in specs]
    sizes = [m.numel() for m in mats]
    assert np.all(np.isfinite(h)) and np.all(h > 0) and np.all(h <= np.log(sizes))
    hb = oracle.block_entropy(h, sizes, bid, wl.n_blocks)
    np.testing.assert_allclose(qp.h_block.cpu().numpy(), hb, rtol=1e-12)
    assert qp.tier.cpu().tolist() == oracle.ewq_tiers(hb)[3].tolist()
    assert all(o["action"] == "sinq" for o in qp.outputs.values()) and len(qp.outputs) == 560
    sample = [i for i, sp in enumerate(specs) if sp.block in (0, 40, 79)]
    h_ref = _oracle_entropies(mats, sample)
    for i in sample:
        np.testing.assert_allclose(h[i], h_ref[i], rtol=1e-10, err_msg=specs[i].name)
    print("[stack70b] oracle entropies of blocks 0, 40, 79 done", flush=True)
    kv = [i for i in sample if specs[i].name.split(".")[-1] in ("k", "v")]
    res = _par.pmap(lambda i: _check_sinq_matrix(_np(mats[i]), qp.outputs[i], wl.iters, wl.bits,
                                                 wl.group), kv)
    iso = [a for a, _ in res]
    e2e = [b for _, b in res]
    rng = np.random.default_rng(2)
    for b in (0, 40, 79):
        for name in ("q", "down"):   # 8192 columns; 28672 columns (512-thread workgroups)
            i = specs.index(next(sp for sp in specs if sp.name == f"b{b}.{name}"))
            if b == 40:
                _check_balance_properties(mats[i], qp.outputs[i], 1e-4)
            rows = np.sort(rng.choice(mats[i].shape[0], 16, replace=False))
            iso.append(_check_rows(mats[i], qp.outputs[i], wl.bits, wl.group, rows))
    bad, tot = _codes.within_budget(iso)
    print(f"[stack70b] codes vs the fp64 definition: {bad} near-tie differences in {tot}", flush=True)
    _codes.within_budget(e2e)
    del qp, mats
    _release()


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_moe_full_configuration():
    """All 24 MoE layers (4,704 matrices, grouped launches of all of them):
    tiers over the 24 layers from the oracle's entropies of every matrix,
    the ternary lowest tier present, and sampled matrices of every layer
    (one attention and two experts) through the oracle."""
    wl, specs, mats = woqdata.generate("moe", device=DEV)
    assert len(mats) == 4704
    qp, tiers = _pass(wl, specs, mats)
    h = qp.h_mat.cpu().numpy()
    bid = [m.block for m in specs]
    sizes = [m.numel() for m in mats]
    print(f"[moe] tiers {tiers}", flush=True)
    hb = oracle.block_entropy(h, sizes, bid, wl.n_blocks)
    assert tiers == qp.tier.cpu().tolist() == oracle.ewq_tiers(hb)[3].tolist()
    h_ref = _oracle_entropies(mats)
    ent_err = max(abs(h[i] / h_ref[i] - 1) for i in range(len(mats)))
    assert ent_err < 1e-10, ent_err
    near = _tier_parity(np.array([h_ref[i] for i in range(len(mats))]), sizes, bid, wl.n_blocks,
                        tiers)
    print(f"[moe] entropies of 4704 matrices: max rel err {ent_err:.2e}; near-boundary layers {near}",
          flush=True)
    acts = qp.action_of_block(tiers)
    assert "ternary" in acts and "sinq" in acts
    rng = np.random.default_rng(3)
    sample = []
    for layer in range(wl.n_blocks):
        idx = [i for i in range(len(specs)) if bid[i] == layer]
        sample += [idx[int(rng.integers(0, 4))]] + [int(i) for i in rng.choice(idx[4:], 2, replace=False)]

    def check(i):
        w = _np(mats[i])
        if acts[bid[i]] == "ternary":
            return "ternary", _check_ternary(w, qp.outputs[i]), None
        return "sinq", *_check_sinq_matrix(w, qp.outputs[i], wl.iters, wl.bits, wl.group)
    res = _par.pmap(check, sample)
    assert {r[0] for r in res} == {"ternary", "sinq"}
    bad, tot = _codes.within_budget([r[1] for r in res])
    _codes.within_budget([r[2] for r in res if r[2] is not None])
    print(f"[moe] {len(sample)} sampled matrices; codes vs the fp64 definitions: {bad} in {tot}",
          flush=True)
    del qp, mats
    _release()


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


def test_balancing_lowers_the_error_on_outlier_channels():
    """The page's case: some columns with much larger variance (and some
    rows).  On such weights K = 16 balancing lowers the reconstruction error
    of every grid and width well below plain group-wise rounding (K = 0),
    by more than a quarter for the affine grids; on i.i.d. weights it changes
    little (the block workload rows of the report)."""
    from weight_only_quantization_softmax_amd import quality
    w = woqdata.channel_matrix(1024, 4096, 5, row_sigma=1.0, col_sigma=1.0, device=DEV)
    rows = quality.matrix_report(w, iters=(0, 16), stds=("centred",), ternary=False)
    by = {(r["scheme"], r["iters"]): r["rel_fro"] for r in rows}
    for bits, group, grid in quality.SCHEMES:
        name = quality.scheme_name(bits, group, grid)
        assert by[(name, 16)] < by[(name, 0)], name
        if grid == "affine":
            assert by[(name, 16)] < 0.75 * by[(name, 0)], (name, by[(name, 16)], by[(name, 0)])
    iid = woqdata.channel_matrix(1024, 4096, 5, row_sigma=0.0, col_sigma=0.0, device=DEV)
    r0 = {(r["scheme"], r["iters"]): r["rel_fro"] for r in
          quality.matrix_report(iid, schemes=((4, 64, "affine"),), iters=(0, 16), stds=("centred",),
                                ternary=False)}
    assert abs(r0[("int4 g64", 16)] / r0[("int4 g64", 0)] - 1) < 0.05


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
