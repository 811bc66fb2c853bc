"""ewq_block_entropy_static (the entropy call with the library's static
scratch array in place of a workspace) through the C ABI, against
ewq_block_entropy on the same inputs: two calls in a row, the second with a
smaller input, every output bit for bit.  The first call has more bf16
matrices than one batch of the static array holds, plus fp32 and strided
matrices; run alone in a fresh process it is also the first call on the
device, where the array's address is looked up."""
import ctypes

import pytest
import torch

import woqdata
import weight_only_quantization_softmax_amd as woq
from weight_only_quantization_softmax_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _static(mats, block_id, n_blocks, x=1.0):
    lib = _lib.load()
    n = len(mats)
    arr = woq._mats(mats)
    out = {"h_mat": torch.full((n,), float("nan"), dtype=torch.float64, device=DEV),
           "h_block": torch.full((n_blocks,), float("nan"), dtype=torch.float64, device=DEV),
           "stats": torch.full((3,), float("nan"), dtype=torch.float64, device=DEV),
           "tier": torch.full((n_blocks,), -1, dtype=torch.int32, device=DEV),
           "order": torch.full((n_blocks,), -1, dtype=torch.int32, device=DEV)}
    bid = (ctypes.c_int32 * n)(*block_id)
    st = lib.ewq_block_entropy_static(arr, n, bid, n_blocks, float(x), out["h_mat"].data_ptr(),
                                      out["h_block"].data_ptr(), out["stats"].data_ptr(),
                                      out["tier"].data_ptr(), out["order"].data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 0, _lib.STATUS.get(st, st)
    return out


def _compare(mats, block_id, n_blocks):
    got = _static(mats, block_id, n_blocks)
    ref = woq.ewq_block_entropy(mats, block_id, n_blocks)
    torch.cuda.synchronize()
    for k in got:
        assert torch.equal(got[k], ref[k]), k
    return got


def test_static_entropy_matches_the_workspace_call_twice():
    # 900 bf16 matrices (more than the 680-odd whose counts one batch of the
    # 32 MiB array holds), fp32 matrices, and column blocks of a fused tensor
    mats, bid = [], []
    for i in range(900):
        mats.append(woqdata.random_matrix(64 + (i % 7) * 16, 256 + 64 * (i % 5), 1000 + i,
                                          std=0.01 + 0.0001 * i).to(DEV))
        bid.append(i % 37)
    for i in range(5):
        mats.append(woqdata.random_matrix(96, 520 + 8 * i, 2000 + i, dtype=torch.float32).to(DEV))
        bid.append(37 + i % 3)
    fused = woqdata.random_matrix(512, 3 * 1024, 3000).to(DEV)
    for j in range(3):
        mats.append(fused[:, 1024 * j:1024 * (j + 1)])
        bid.append(40)
    first = _compare(mats, bid, 41)
    assert torch.all(torch.isfinite(first["h_mat"]))
    # the second call, smaller: a few matrices in two blocks
    small = [woqdata.random_matrix(128, 512, 4000 + i, std=0.02 + 0.01 * i).to(DEV) for i in range(5)]
    second = _compare(small, [0, 0, 1, 1, 1], 2)
    assert second["h_mat"].numel() == 5
