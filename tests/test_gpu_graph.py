"""Graph capture: every library call can be captured into a HIP graph (its
descriptor tables travel in kernel arguments while the stream captures),
and an untiered pass is captured whole.  Each test replays a graph several
times with the program's own eager work and synchronisations in between
(the outputs overwritten, other library calls run) and checks every replay
against the eager result, bit for bit."""
import ctypes

import pytest
import torch

import woqdata
import weight_only_quantization_softmax_amd as woq
from weight_only_quantization_softmax_amd import _lib
from weight_only_quantization_softmax_amd.pipeline import QuantPass

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _tensors(outputs):
    return {(i, k): v for i, o in outputs.items() for k, v in o.items() if isinstance(v, torch.Tensor)}


def _bits(t):
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


@pytest.mark.parametrize("name", ["single", "block"])
def test_pass_graph_replays_match_the_eager_pass(name):
    wl, specs, mats = woqdata.generate(name, device=DEV)
    qp = QuantPass(mats, [m.block for m in specs], wl.n_blocks, iters=wl.iters, bits=wl.bits,
                   group=wl.group, tiered=wl.tiered, actions=(wl.low_tier, wl.mid_tier, wl.high_tier))
    qp.run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in _tensors(qp.outputs).items()}
    ref_h = qp.h_mat.clone()
    g = qp.graph()
    other = woqdata.random_matrix(300, 1024, 9).to(DEV)
    for rep in range(3):
        for v in _tensors(qp.outputs).values():
            v.fill_(7 if v.dtype == torch.uint8 else -1)
        qp.h_mat.fill_(float("nan"))
        woq.sinq_balance([other], 4)             # other library work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _tensors(qp.outputs)
        assert got.keys() == ref.keys()
        for k in ref:
            assert torch.equal(_bits(got[k]), _bits(ref[k])), (rep, k)
        assert torch.equal(qp.h_mat, ref_h), rep


def test_single_calls_captured():
    """quant_pack_groupwise, sinq_balance and ewq_block_entropy_static (the
    entry point that allocates nothing) captured one by one."""
    m = [woqdata.random_matrix(256, 2048, 11).to(DEV), woqdata.random_matrix(64, 14336, 12).to(DEV)]
    s, t = woq.sinq_balance(m, 6)
    codes, scales, zeros = woq.quant_pack_groupwise(m, 4, 64, row_scale=s, col_scale=t)
    h = woq.ewq_block_entropy(m, [0, 1], 2)
    torch.cuda.synchronize()
    ref = [x.clone() for x in s + t + codes + scales + zeros] + [h["h_mat"].clone(), h["tier"].clone()]
    ws_s = torch.empty(woq.workspace_size(_lib.OP_SINQ, m), dtype=torch.uint8, device=DEV)
    ws_q = torch.empty(woq.workspace_size(_lib.OP_QUANT, m, 64), dtype=torch.uint8, device=DEV)
    h_mat = torch.empty(2, dtype=torch.float64, device=DEV)
    h_blk = torch.empty(2, dtype=torch.float64, device=DEV)
    stats = torch.empty(3, dtype=torch.float64, device=DEV)
    tier = torch.empty(2, dtype=torch.int32, device=DEV)
    order = torch.empty(2, dtype=torch.int32, device=DEV)
    arr = woq._mats(m)
    bid = (ctypes.c_int32 * 2)(0, 1)
    lib = _lib.load()
    # the first call on the device, which locates the static array, is made
    # eagerly; it already matches the workspace call
    cur = torch.cuda.current_stream().cuda_stream
    assert lib.ewq_block_entropy_static(arr, 2, bid, 2, 1.0, h_mat.data_ptr(), h_blk.data_ptr(),
                                        stats.data_ptr(), tier.data_ptr(), order.data_ptr(), cur) == 0
    torch.cuda.synchronize()
    assert torch.equal(h_mat, ref[-2]) and torch.equal(tier, ref[-1])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cur = torch.cuda.current_stream().cuda_stream
        woq.sinq_balance(m, 6, row_scale=s, col_scale=t, ws=ws_s)
        woq.quant_pack_groupwise(m, 4, 64, row_scale=s, col_scale=t, codes=codes, scales=scales,
                                 zeros=zeros, ws=ws_q)
        assert lib.ewq_block_entropy_static(arr, 2, bid, 2, 1.0, h_mat.data_ptr(), h_blk.data_ptr(),
                                            stats.data_ptr(), tier.data_ptr(), order.data_ptr(),
                                            cur) == 0
    for rep in range(3):
        for x in s + t + scales + [h_mat]:
            x.fill_(float("nan"))
        for x in codes + zeros:
            x.fill_(0xEE)
        tier.fill_(-5)
        woq.ewq_block_entropy([woqdata.random_matrix(32, 512, 13).to(DEV)])   # eager work between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = s + t + codes + scales + zeros + [h_mat, tier]
        for a, b in zip(got, ref):
            assert torch.equal(_bits(a), _bits(b)), rep
