"""Seeded synthetic weight matrices for the quantisation pass.

This module only draws random numbers and arranges them into the shapes of
the workloads; it holds none of the method's arithmetic (no entropy, no
scaling, no rounding to codes).  Both the CPU oracle and the HIP path consume
the tensors it returns, so it is the single shared input source.

Workloads (rows x cols is out_features x in_features, row-major):

* ``single``   one fp32 256x512 matrix, N(0, 0.02^2) with 1% of the entries
               (distinct, uniformly chosen) multiplied by 20.
* ``block``    one Llama-style transformer block in bf16: d=4096, GQA kv dim
               1024, SwiGLU FFN 14336; N(0, 0.02^2) plus 0.1% entries x10.
* ``stack8b``  32 blocks of the ``block`` shapes (Llama-3.1-8B-shaped linear
               weights, 6.98e9 bf16 values); per-block std ~ U(0.01, 0.04).
* ``stack70b`` 80 blocks with d=8192, kv 1024, FFN 28672; same distribution
               as ``stack8b``.
* ``moe``      24 layers, each with attention at d=2048 / kv 512 (std 0.02)
               and 64 experts (gate/up 1408x2048, down 2048x1408) whose std is
               0.02*exp(0.5*z), z ~ N(0,1) (log-normal around 0.02); no
               outliers.  A layer is one block (4 + 192 matrices).

Seeding.  ``single`` draws from ``torch.Generator('cpu').manual_seed(0)``.
Every other matrix uses its own generator on the requested device seeded with
``(config << 40) | (block << 20) | index``; the per-block / per-expert std
draws come from a CPU generator seeded ``(config << 40) | (0xFFFFF << 20)``.
The values therefore depend on the device the weights are drawn on (torch's
CPU and GPU generators differ); the std draws do not.  bf16 weights are drawn
in fp32 and rounded to nearest-even.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import torch

__all__ = [
    "MatSpec", "Workload", "WORKLOADS", "workload", "weights", "generate",
    "draw_matrix", "random_matrix", "channel_matrix",
]


@dataclasses.dataclass(frozen=True)
class MatSpec:
    name: str          # e.g. "b3.gate" or "l2.e17.down"
    block: int         # EWQ block (transformer block / MoE layer) index
    index: int         # position inside the block (seed component)
    rows: int
    cols: int
    std: float
    outlier_frac: float
    outlier_mult: float
    expert: int = -1   # MoE expert id, -1 for attention / dense weights

    @property
    def numel(self) -> int:
        return self.rows * self.cols


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    config_id: int
    dtype: torch.dtype
    n_blocks: int
    mats: tuple            # tuple[MatSpec, ...]
    # pipeline parameters of the workload (what the pass is asked to do)
    iters: int             # Sinkhorn iterations
    bits: int              # low-bit code width for the Sinkhorn tier
    group: int             # group size along columns
    tiered: bool           # EWQ tiering decides the action per block
    low_tier: str          # action for the lowest-entropy tier: "sinq" or "ternary"
    mid_tier: str          # action for the middle tier: "int8row" or "sinq"
    high_tier: str         # action for the top tier: "keep" or "sinq"
    x: float = 1.0         # EWQ threshold multiplier

    @property
    def numel(self) -> int:
        return sum(m.numel for m in self.mats)

    @property
    def bytes(self) -> int:
        return self.numel * (4 if self.dtype == torch.float32 else 2)


def _llama_block(b: int, d: int, kv: int, ffn: int, std: float,
                 frac: float, mult: float) -> List[MatSpec]:
    shapes = [("q", d, d), ("k", kv, d), ("v", kv, d), ("o", d, d),
              ("gate", ffn, d), ("up", ffn, d), ("down", d, ffn)]
    return [MatSpec(f"b{b}.{n}", b, k, r, c, std, frac, mult)
            for k, (n, r, c) in enumerate(shapes)]


def _std_generator(config_id: int) -> torch.Generator:
    g = torch.Generator("cpu")
    g.manual_seed((config_id << 40) | (0xFFFFF << 20))
    return g


def _make(name: str) -> Workload:
    if name == "single":
        mats = (MatSpec("w", 0, 0, 256, 512, 0.02, 0.01, 20.0),)
        return Workload(name, 1, torch.float32, 1, mats, 16, 4, 64, False,
                        "sinq", "sinq", "sinq")
    if name == "block":
        mats = tuple(_llama_block(0, 4096, 1024, 14336, 0.02, 0.001, 10.0))
        return Workload(name, 2, torch.bfloat16, 1, mats, 16, 4, 64, False,
                        "sinq", "sinq", "sinq")
    if name in ("stack8b", "stack70b"):
        cid, nb = (3, 32) if name == "stack8b" else (4, 80)
        d, kv, ffn = (4096, 1024, 14336) if name == "stack8b" else (8192, 1024, 28672)
        g = _std_generator(cid)
        stds = (0.01 + 0.03 * torch.rand(nb, generator=g, dtype=torch.float64)).tolist()
        mats = []
        for b in range(nb):
            mats += _llama_block(b, d, kv, ffn, stds[b], 0.001, 10.0)
        if name == "stack8b":
            return Workload(name, cid, torch.bfloat16, nb, tuple(mats), 16, 4, 64,
                            True, "sinq", "int8row", "keep")
        return Workload(name, cid, torch.bfloat16, nb, tuple(mats), 24, 3, 128,
                        False, "sinq", "sinq", "sinq")
    if name == "moe":
        cid, nl, ne = 5, 24, 64
        g = _std_generator(cid)
        z = torch.randn(nl * ne, generator=g, dtype=torch.float64)
        stds = (0.02 * torch.exp(0.5 * z)).tolist()
        mats = []
        for l in range(nl):
            for k, (n, r, c) in enumerate([("q", 2048, 2048), ("k", 512, 2048),
                                           ("v", 512, 2048), ("o", 2048, 2048)]):
                mats.append(MatSpec(f"l{l}.{n}", l, k, r, c, 0.02, 0.0, 1.0))
            for e in range(ne):
                s = stds[l * ne + e]
                for j, (n, r, c) in enumerate([("gate", 1408, 2048), ("up", 1408, 2048),
                                               ("down", 2048, 1408)]):
                    mats.append(MatSpec(f"l{l}.e{e}.{n}", l, 4 + 3 * e + j, r, c,
                                        s, 0.0, 1.0, expert=e))
        return Workload(name, cid, torch.bfloat16, nl, tuple(mats), 16, 4, 64, True,
                        "ternary", "sinq", "sinq")
    raise KeyError(name)


WORKLOADS = ("single", "block", "stack8b", "stack70b", "moe")


def workload(name: str) -> Workload:
    return _make(name)


def _seed(config_id: int, block: int, index: int) -> int:
    return (config_id << 40) | (block << 20) | index


def draw_matrix(rows: int, cols: int, std: float, outlier_frac: float,
                outlier_mult: float, dtype: torch.dtype, seed: int,
                device="cpu") -> torch.Tensor:
    """N(0, std^2) weights with round(frac*n) distinct entries multiplied."""
    device = torch.device(device)
    g = torch.Generator(device.type)
    g.manual_seed(int(seed))
    w = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    w.mul_(std)
    n = rows * cols
    k = int(round(outlier_frac * n))
    if k > 0:
        idx = torch.randperm(n, generator=g, device=device)[:k]
        flat = w.view(-1)
        flat[idx] = flat[idx] * outlier_mult
    return w.to(dtype)


def weights(spec: MatSpec, wl: Workload, device="cpu") -> torch.Tensor:
    if wl.name == "single":
        g = torch.Generator("cpu")
        g.manual_seed(0)
        w = spec.std * torch.randn(spec.rows, spec.cols, generator=g)
        n = spec.numel
        k = int(round(spec.outlier_frac * n))
        idx = torch.randperm(n, generator=g)[:k]
        w.view(-1)[idx] *= spec.outlier_mult
        return w.to(device)
    return draw_matrix(spec.rows, spec.cols, spec.std, spec.outlier_frac,
                       spec.outlier_mult, wl.dtype,
                       _seed(wl.config_id, spec.block, spec.index), device)


def generate(name: str, device="cpu", blocks: Optional[Sequence[int]] = None):
    """Return (workload, [MatSpec], [tensor]) for the chosen blocks (all if None)."""
    wl = workload(name)
    specs = [m for m in wl.mats if blocks is None or m.block in set(blocks)]
    return wl, specs, [weights(m, wl, device) for m in specs]


def random_matrix(rows: int, cols: int, seed: int, dtype=torch.bfloat16,
                  std: float = 0.02, outlier_frac: float = 0.001,
                  outlier_mult: float = 10.0, device="cpu") -> torch.Tensor:
    """A free-shape matrix with the workloads' value distribution (test sizes)."""
    return draw_matrix(rows, cols, std, outlier_frac, outlier_mult, dtype,
                       (7 << 40) | (int(seed) & ((1 << 40) - 1)), device)


def channel_matrix(rows: int, cols: int, seed: int, dtype=torch.bfloat16, std: float = 0.02,
                   row_sigma: float = 1.0, col_sigma: float = 1.0, device="cpu") -> torch.Tensor:
    """Weights with outlier channels: N(0, std^2) draws whose rows and columns
    are multiplied by random log-normal factors exp(row_sigma a_i) and
    exp(col_sigma b_j), a, b ~ N(0, 1) (some rows and some columns much larger
    than the rest).  Random draws only; one CPU generator, so the values do
    not depend on the device."""
    g = torch.Generator("cpu")
    g.manual_seed((6 << 40) | (int(seed) & ((1 << 40) - 1)))
    w = torch.randn(rows, cols, generator=g, dtype=torch.float32) * std
    a = torch.randn(rows, generator=g, dtype=torch.float32)
    b = torch.randn(cols, generator=g, dtype=torch.float32)
    w = w * torch.exp(row_sigma * a)[:, None] * torch.exp(col_sigma * b)[None, :]
    return w.to(dtype).to(device)


def _check() -> None:  # shapes sanity, used by tests
    wl = workload("stack8b")
    assert wl.numel == 6_979_321_856, wl.numel
    assert math.isclose(wl.bytes / 1e9, 13.958643712)
