"""Data-free quality report: how well the quantised weights reconstruct W.

SINQ's claim is that balancing rows and columns before rounding spreads the
rounding error more evenly and lowers it ([SINQ] "Huawei gioi thieu SINQ"
(asiadaily.org), sections "Dinh ty le tren hai truc" and "Chuan hoa
Sinkhorn Knopp").  This measures it on the weights alone, with no data: each
matrix is balanced for K iterations (with the centred std, and with the
uncentred root mean square for comparison), quantised and packed, then
decoded with dequant_unpack, all through the library; the report gives, per
matrix, scheme, K and std, the relative Frobenius error ||W - W'|| / ||W||
and the largest absolute error, both computed in fp64 on the device.  K = 0
is plain
group-wise RTN (s = t = 1).  Each width is reported on the affine grid
(int, scale and zero-point per group) and on the normal-quantile code book
(nf, the nearest of 2^b levels scaled by the group's largest |x|), the
non-uniform option of [SINQ] section "Tiet kiem bo nho, toc do va chat
luong trong thu nghiem".  Ternary codes ([BitNet] "Khung Nguon
BitNet.cpp" (unite.ai), "He Thong Trong So Ternary") use the per-row scale
and no balancing.

    python -m weight_only_quantization_softmax_amd.quality --workload block --blocks 0
    python -m weight_only_quantization_softmax_amd.quality --channels 1 1 --shape 1024 4096

The second form reports on weights with outlier channels (woqdata's
channel_matrix: rows and columns scaled by random log-normal factors), the
case the page names: some rows with outliers, some columns with larger
variance.
"""
from __future__ import annotations

import argparse
import json
import sys
from typing import Dict, List, Sequence, Tuple

import torch

from . import (dequant_codebook, dequant_unpack, quant_pack_codebook, quant_pack_groupwise,
               sinq_balance, ternary_pack)

# (bits, group, grid): grid "affine" (integer codes) or "normal" (the
# normal-quantile code book)
SCHEMES: Tuple[Tuple[int, int, str], ...] = ((4, 64, "affine"), (3, 128, "affine"),
                                             (4, 64, "normal"), (3, 128, "normal"))
ITERS: Tuple[int, ...] = (0, 4, 16, 24)
# the std used by the balancing: centred (the pass's reading) or the
# uncentred root mean square
STDS: Tuple[str, ...] = ("centred", "rms")


def _errors(w: torch.Tensor, wq: torch.Tensor) -> Dict[str, float]:
    a = w.double()
    d = wq.double() - a
    return {"rel_fro": (torch.linalg.vector_norm(d) / torch.linalg.vector_norm(a)).item(),
            "max_abs": d.abs().max().item()}


def scheme_name(bits: int, group: int, grid: str) -> str:
    return f"{'int' if grid == 'affine' else 'nf'}{bits} g{group}"


def _round_trip(w, bits, group, grid, s, t):
    shape = tuple(w.shape)
    if grid == "affine":
        codes, scales, zeros = quant_pack_groupwise([w], bits, group, row_scale=s, col_scale=t)
        return dequant_unpack([shape], codes, scales, bits, group, zeros=zeros, row_scale=s,
                              col_scale=t, out_dtype=torch.float32)[0]
    codes, scales = quant_pack_codebook([w], bits, group, row_scale=s, col_scale=t)
    return dequant_codebook([shape], codes, scales, bits, group, row_scale=s, col_scale=t,
                            out_dtype=torch.float32)[0]


def matrix_report(w: torch.Tensor, schemes: Sequence[Tuple[int, int, str]] = SCHEMES,
                  iters: Sequence[int] = ITERS, ternary: bool = True,
                  stds: Sequence[str] = STDS) -> List[dict]:
    """Rows of the report for one device-resident matrix (bf16 or fp32):
    one per (scheme, K, std) with K > 0, one per scheme at K = 0 (plain RTN,
    std "none"), and the ternary row."""
    rows = []
    shape = tuple(w.shape)
    for bits, group, grid in schemes:
        for k in iters:
            for std in (stds if k else ("none",)):
                s, t = sinq_balance([w], k, rms=(std == "rms"))
                wq = _round_trip(w, bits, group, grid, s, t)
                rows.append({"scheme": scheme_name(bits, group, grid), "iters": k, "std": std,
                             **_errors(w, wq)})
    if ternary:
        codes, beta = ternary_pack([w])
        wq = dequant_unpack([shape], codes, [beta[0]], 2, 0, out_dtype=torch.float32)[0]
        rows.append({"scheme": "ternary", "iters": 0, "std": "none", **_errors(w, wq)})
    return rows


def main(argv=None) -> int:
    import woqdata

    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="block")
    ap.add_argument("--blocks", type=int, nargs="*", default=[0])
    ap.add_argument("--matrices", nargs="*", default=None,
                    help="matrix name suffixes to include (e.g. k v gate); all if omitted")
    ap.add_argument("--channels", type=float, nargs=2, default=None, metavar=("ROW_SIGMA", "COL_SIGMA"),
                    help="report on a channel_matrix with these log-normal spreads instead")
    ap.add_argument("--shape", type=int, nargs=2, default=(1024, 4096))
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args(argv)
    torch.cuda.set_device(0)
    if args.channels is not None:
        w = woqdata.channel_matrix(*args.shape, args.seed, row_sigma=args.channels[0],
                                   col_sigma=args.channels[1], device="cuda")
        name = f"channels(row {args.channels[0]}, col {args.channels[1]})"
        for r in matrix_report(w):
            print(json.dumps({"matrix": name, "shape": list(w.shape), **r}), flush=True)
        return 0
    wl, specs, mats = woqdata.generate(args.workload, device="cuda", blocks=args.blocks)
    for spec, w in zip(specs, mats):
        if args.matrices and spec.name.split(".")[-1] not in args.matrices:
            continue
        for r in matrix_report(w):
            print(json.dumps({"matrix": spec.name, "shape": list(w.shape), **r}), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
