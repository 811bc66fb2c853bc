"""Argument checks of the Python binding that run before any HIP call (no GPU).

The library takes raw pointers: a host tensor, a buffer list shorter than the
matrix list or an undersized output would make its kernels read or write
outside what the caller owns.  The binding must refuse all of these with a
Python exception before anything is enqueued.
"""
import pytest
import torch

import weight_only_quantization_softmax_amd as woq
from weight_only_quantization_softmax_amd.pipeline import QuantPass


def _m(r=4, c=64, dt=torch.bfloat16):
    return torch.zeros(r, c, dtype=dt)


def test_empty_matrix_lists_are_rejected():
    with pytest.raises(ValueError, match="at least one"):
        woq.ewq_block_entropy([])
    with pytest.raises(ValueError, match="at least one"):
        woq.sinq_balance([], 4)
    with pytest.raises(ValueError, match="at least one"):
        woq.quant_pack_groupwise([], 4, 64)
    with pytest.raises(ValueError, match="at least one"):
        woq.quant_pack_codebook([], 4, 64)
    with pytest.raises(ValueError, match="at least one"):
        woq.ternary_pack([])
    with pytest.raises(ValueError, match="at least one"):
        woq.df11_exponent_histogram([])
    with pytest.raises(ValueError, match="at least one"):
        woq.df11_decode([])
    with pytest.raises(ValueError, match="at least one"):
        woq.dequant_unpack([], [], [], 4, 64)
    with pytest.raises(ValueError, match="at least one"):
        woq.dequant_codebook([(0, 64)], [], [], 4, 64)
    with pytest.raises(ValueError, match="at least one"):
        woq.workspace_size(0, [])


@pytest.mark.parametrize("shape", [(0, 64), (4, 0)])
def test_empty_matrices_are_rejected(shape):
    with pytest.raises(ValueError, match="empty matrix"):
        woq.sinq_balance([_m(*shape)], 4)
    with pytest.raises(ValueError, match="empty matrix"):
        woq.quant_pack_groupwise([_m(*shape)], 4, 64)


def test_host_tensors_never_reach_the_library():
    for call in (lambda: woq.ewq_block_entropy([_m()]),
                 lambda: woq.sinq_balance([_m()], 4),
                 lambda: woq.quant_pack_groupwise([_m()], 4, 64),
                 lambda: woq.quant_pack_codebook([_m()], 4, 64),
                 lambda: woq.ternary_pack([_m()]),
                 lambda: woq.df11_exponent_histogram([_m()]),
                 lambda: QuantPass([_m()], [0], 1, iters=4, bits=4, group=64)):
        with pytest.raises(ValueError, match="on a GPU"):
            call()
    # decoders: host inputs, or no tensor at all to take the device from
    codes, scales, zeros = [torch.zeros(4, 32, dtype=torch.uint8)], [torch.zeros(4, 1)], \
        [torch.zeros(4, 1, dtype=torch.uint8)]
    with pytest.raises(ValueError, match="on a GPU"):
        woq.dequant_unpack([(4, 64)], codes, scales, 4, 64, zeros=zeros)
    with pytest.raises(ValueError, match="no GPU tensor"):
        woq.dequant_unpack([(4, 64)], None, None, 4, 64)


def test_buffer_lists_match_the_matrices():
    mats = [_m(), _m(8, 128)]
    with pytest.raises(ValueError, match="1 tensors for 2 matrices"):
        woq.sinq_balance(mats, 4, row_scale=[torch.zeros(4)])
    with pytest.raises(ValueError, match="1 tensors for 2 matrices"):
        woq.quant_pack_groupwise(mats, 4, 64, codes=[torch.zeros(4, 32, dtype=torch.uint8)])
    with pytest.raises(ValueError, match="ids for 2 matrices"):
        woq.ewq_block_entropy(mats, block_id=[0])


def test_undersized_or_mistyped_buffers_are_rejected():
    m = [_m(4, 128)]
    # int4 codes of a 4 x 128 matrix: 4 * 64 bytes
    with pytest.raises(ValueError, match="255 elements, 256 needed"):
        woq.quant_pack_groupwise(m, 4, 64, codes=[torch.zeros(255, dtype=torch.uint8)])
    with pytest.raises(TypeError, match="expected torch.uint8"):
        woq.quant_pack_groupwise(m, 4, 64, codes=[torch.zeros(4, 64, dtype=torch.int8)])
    # scales: one per group of 64 -> 4 x 2
    with pytest.raises(ValueError, match="7 elements, 8 needed"):
        woq.quant_pack_groupwise(m, 4, 64, scales=[torch.zeros(7)])
    with pytest.raises(ValueError, match="must be contiguous"):
        woq.sinq_balance(m, 4, col_scale=[torch.zeros(256)[::2]])
    with pytest.raises(ValueError, match="3 elements, 4 needed"):
        woq.ternary_pack(m, row_scale=[torch.zeros(3)])
    with pytest.raises(ValueError, match="out: tensors do not have the given shapes"):
        woq.dequant_unpack([(4, 128)], [torch.zeros(4, 64, dtype=torch.uint8)],
                           [torch.zeros(4, 2)], 4, 64, out=[torch.zeros(4, 64)])
    with pytest.raises(ValueError, match="511 elements, 512 needed"):
        woq.df11_exponent_histogram([_m(), _m()], hist=torch.zeros(511, dtype=torch.int32))
