"""The seeded synthetic workloads have the stated shapes and sizes."""
import torch

import woqdata


def test_workload_sizes():
    woqdata._check()
    sizes = {n: woqdata.workload(n).numel for n in woqdata.WORKLOADS}
    assert sizes["single"] == 131_072
    assert sizes["block"] == 218_103_808
    assert sizes["stack8b"] == 6_979_321_856
    assert sizes["stack70b"] == 68_451_041_280
    assert sizes["moe"] == 13_539_213_312
    assert len(woqdata.workload("moe").mats) == 24 * (4 + 64 * 3)


def test_single_matrix_recipe():
    wl, specs, ws = woqdata.generate("single")
    w = ws[0]
    assert w.dtype == torch.float32 and w.shape == (256, 512)
    # 1% of entries are x20 outliers: about 1311 entries beyond 4 sigma
    assert 1000 < int((w.abs() > 0.1).sum()) < 1400


def test_seeded_and_distinct():
    a = woqdata.random_matrix(64, 128, 1)
    b = woqdata.random_matrix(64, 128, 1)
    c = woqdata.random_matrix(64, 128, 2)
    assert torch.equal(a, b) and not torch.equal(a, c)
    assert a.dtype == torch.bfloat16


def test_block_std_draws():
    wl = woqdata.workload("stack8b")
    stds = sorted({m.std for m in wl.mats})
    assert len(stds) == 32 and 0.01 <= stds[0] and stds[-1] <= 0.04
    moe = woqdata.workload("moe")
    e = {(m.block, m.expert): m.std for m in moe.mats if m.expert >= 0}
    assert len(e) == 24 * 64
