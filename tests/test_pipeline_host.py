"""Host-side logic of the pass's dispatch (no GPU): how the Sinkhorn step of
a tier is split into two concurrent calls."""
import torch

from weight_only_quantization_softmax_amd import _lib
from weight_only_quantization_softmax_amd.pipeline import QuantPass, _wave_form


def _m(r, c, dt=torch.bfloat16):
    return torch.empty(r, c, dtype=dt)   # shapes and dtypes only


def test_wave_form_limits():
    assert _wave_form(_m(4, 4096)) and not _wave_form(_m(4, 4104))
    assert _wave_form(_m(4, 1536, torch.float32)) and not _wave_form(_m(4, 1544, torch.float32))


def test_llama_block_splits_wide_rows_with_the_shared_plan():
    mats = [_m(4096, 4096), _m(1024, 4096), _m(1024, 4096), _m(4096, 4096),
            _m(14336, 4096), _m(14336, 4096), _m(4096, 14336)]
    first, second, flags = QuantPass._sinq_split(mats)
    assert first == [0, 1, 2, 3, 4, 5] and second == [6]
    assert flags == _lib.WOQ_SINQ_SHARED


def test_single_form_tiers_split_by_width_without_flags():
    # MoE layer: 2048-column matrices hold most bytes; 1408-column ones go second
    mats = [_m(2048, 2048), _m(512, 2048), _m(1408, 2048), _m(2048, 1408), _m(1408, 2048)]
    first, second, flags = QuantPass._sinq_split(mats)
    assert first == [0, 1, 2, 4] and second == [3] and flags == 0
    # 70B block: all rows wider than one wave; 8192-column matrices hold most bytes
    mats = [_m(8192, 8192), _m(28672, 8192), _m(28672, 8192), _m(8192, 28672)]
    first, second, flags = QuantPass._sinq_split(mats)
    assert first == [0, 1, 2] and second == [3] and flags == 0


def test_one_width_is_one_call():
    assert QuantPass._sinq_split([_m(64, 1024), _m(128, 1024)]) is None
    assert QuantPass._sinq_split([_m(64, 1024)]) is None
    # same width, different dtypes: two launch classes, split
    first, second, flags = QuantPass._sinq_split([_m(64, 1024), _m(64, 1024, torch.float32)])
    assert sorted(first + second) == [0, 1] and flags == 0
