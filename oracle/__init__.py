"""CPU oracle for the calibration-free weight-quantisation pass.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously correct
reference written from the pages' definitions.  Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path (the HIP library and its Python binding) never does, and the
oracle imports nothing from the product path.  Its only inputs are tensors
from the neutral generator ``woqdata`` (copied to the host) or hand-made
arrays.

Sources (cited by page title and section; the pages are Vietnamese):

* [EWQ]  "Giải mã EWQ & FastEWQ: Lượng tử hóa LLM 'thông minh' hơn, nhẹ hơn
  mà không cần hy sinh hiệu suất" (2kvn.com), section "EWQ hoạt động như thế
  nào?" (how EWQ works): step 1 "Phân tích Entropy của từng Khối" (per-block
  entropy), step 2 "Tiêu chí lựa chọn khối để Lượng tử hóa" (block
  selection criterion) and step 3 (budgeted placement in the cluster,
  "Algorithm 1").
* [SINQ] "Huawei giới thiệu SINQ: phương pháp lượng tử hóa mã nguồn mở giúp LLM
  hoạt động hiệu quả hơn" (asiadaily.org), sections "Định tỷ lệ trên hai trục"
  (dual-axis scaling) and "Chuẩn hóa Sinkhorn Knopp" (Sinkhorn-Knopp
  normalisation); the 4-bit / 3-bit integer targets in "Vì sao SINQ quan
  trọng…" and "Những gì nhà phát triển có thể sử dụng ngay hôm nay"; the
  non-uniform option in "Tiết kiệm bộ nhớ, tốc độ và chất lượng trong thử
  nghiệm" (module ``oracle.codebook``).
* [BitNet] "Khung Nguồn BitNet.cpp Của Microsoft Đưa Mô Hình Ngôn Ngữ Lớn 1-Bit
  Đến Thiết Bị Địa Phương" (unite.ai), sections "Hệ Thống Trọng Số Ternary"
  (the {-1, 0, +1} weight set) and "Lượng Tử Hóa Nhóm và Chuẩn Hóa" (groups
  are quantised independently).
* [DF11] "DFloat11: Nén suy luận GPU không mất dữ liệu, giảm LLM xuống còn 70%
  kích thước" (vi.news.hada.io): the lossless exponent code for the blocks
  kept in bf16 (module ``oracle.df11``).

Precision.  Everything is fp64 except where floating point decides an integer
code: there the oracle takes the decision in fp32, with the same sequence of
correctly rounded IEEE operations (+, -, *, /, round-half-even) that the
kernels use, so codes compare bit-exactly.  An fp64 variant of the quantiser
is kept for the error-bound pins and for end-to-end comparisons under the
near-tie rule.

Parity pins: every function here is pinned by a ``-m "not gpu"`` test against
closed forms, library routines, brute force (mpmath / exact fractions) or hand
fixtures under ``tests/golden``.  No function is left "parity unpinned".
"""
from .ewq import matrix_entropy, block_entropy, ewq_tiers, ewq_order, ewq_budget
from .sinq import sinkhorn_std, line_std
from .rtn import (quantize_groupwise_f32, quantize_groupwise_f64, pack_codes,
                  unpack_codes, dequantize_f32, near_tie_mask)
from .ternary import (ternary_quantize, ternary_dequantize, ternary_quantize_f64,
                      ternary_near_tie_mask)

__all__ = [
    "matrix_entropy", "block_entropy", "ewq_tiers", "ewq_order", "ewq_budget",
    "sinkhorn_std", "line_std",
    "quantize_groupwise_f32", "quantize_groupwise_f64", "pack_codes",
    "unpack_codes", "dequantize_f32", "near_tie_mask",
    "ternary_quantize", "ternary_dequantize", "ternary_quantize_f64",
    "ternary_near_tie_mask",
]
from . import df11  # noqa: F401
from . import codebook  # noqa: F401
