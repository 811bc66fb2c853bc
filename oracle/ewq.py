"""EWQ entropy scoring and tiering (oracle, fp64).  Test infrastructure only.

[EWQ] step 1: each weight matrix is flattened, turned into a probability
distribution by softmax, and scored by its Shannon entropy; a block's entropy
is the mean of its matrices' entropies weighted by matrix size.
[EWQ] step 2: blocks are ordered by ascending entropy; with the mean mu_H and
standard deviation sigma_H of the block entropies, T = mu_H - X * sigma_H
(X = 1 by default); H <= T -> aggressive quantisation (tier 1),
T < H < mu_H -> moderate (tier 2), H >= mu_H -> kept (tier 3).

Readings where the page is silent: natural logarithm (nats); one softmax over
all rows*cols entries with the raw weights as logits; "size" = element count;
sigma_H is the population standard deviation over all blocks; when two rules
match (sigma_H = 0 makes T = mu_H) the first rule listed wins.
"""
from __future__ import annotations

import numpy as np


def matrix_entropy(w) -> float:
    """Shannon entropy (nats) of softmax(flatten(w)).

    Written as the definition: p = exp(w) / sum(exp(w)) (evaluated with the
    maximum subtracted, which leaves p unchanged), H = -sum p ln p, with the
    convention 0 ln 0 = 0.  Any non-finite weight gives NaN.
    """
    x = np.asarray(w, dtype=np.float64).ravel()
    if x.size == 0:
        raise ValueError("entropy of an empty matrix is undefined")
    if not np.all(np.isfinite(x)):
        return float("nan")
    e = np.exp(x - x.max())
    p = e / e.sum()
    p = p[p > 0]
    return float(-np.sum(p * np.log(p)))


def block_entropy(h_mat, sizes, block_id, n_blocks: int) -> np.ndarray:
    """Size-weighted mean of matrix entropies per block: sum n_m H_m / sum n_m."""
    h_mat = np.asarray(h_mat, dtype=np.float64)
    sizes = np.asarray(sizes, dtype=np.float64)
    block_id = np.asarray(block_id, dtype=np.int64)
    out = np.empty(n_blocks, dtype=np.float64)
    for b in range(n_blocks):
        sel = block_id == b
        if not sel.any():
            raise ValueError(f"block {b} has no matrices")
        out[b] = np.sum(sizes[sel] * h_mat[sel]) / np.sum(sizes[sel])
    return out


def ewq_tiers(h_block, x: float = 1.0, ddof: int = 0):
    """(mu, sigma, T, tiers) with tiers in {1, 2, 3} as in [EWQ] step 2."""
    h = np.asarray(h_block, dtype=np.float64)
    mu = float(np.mean(h))
    sigma = float(np.sqrt(np.sum((h - mu) ** 2) / (h.size - ddof))) if h.size > ddof else 0.0
    t = mu - x * sigma
    tiers = np.where(h <= t, 1, np.where(h < mu, 2, 3)).astype(np.int32)
    return mu, sigma, t, tiers


def ewq_order(h_block) -> np.ndarray:
    """Blocks in ascending entropy order, ties broken by block index."""
    h = np.asarray(h_block, dtype=np.float64)
    return np.array(sorted(range(h.size), key=lambda b: (h[b], b)), dtype=np.int32)


def ewq_budget(h_block, level_bytes, level0, budget: int):
    """[EWQ] step 3 (budgeted placement, "Algorithm 1"): adjust the tiers'
    precision levels to a memory budget.

    ``level_bytes[b][l]`` is block b's storage at level l, levels in
    ascending size (e.g. 0 ternary, 1 int4 after balancing, 2 int8 per row,
    3 kept bf16); ``level0`` are the levels the tiers give.  The page says
    that spare room goes to promoting the highest-entropy quantised blocks
    to higher precision, and that a shortfall is met by demoting the
    lowest-entropy blocks to lower precision.  Reading taken here, one level
    at a time:

    * total <= budget: repeatedly promote, by one level, the block of
      highest entropy (ties: lower index) among those below the top level
      whose promotion still fits; stop when none fits;
    * total > budget: repeatedly demote, by one level, the block of lowest
      entropy (ties: lower index) among those above the bottom level; stop
      when the total fits or nothing can be demoted.

    Returns (levels, total bytes, fits).
    """
    h = [float(v) for v in h_block]
    lb = [[int(x) for x in row] for row in level_bytes]
    lev = [int(v) for v in level0]
    top = [len(row) - 1 for row in lb]
    total = sum(lb[b][lev[b]] for b in range(len(h)))
    if total <= budget:
        while True:
            best = None
            for b in range(len(h)):
                if lev[b] < top[b] and total - lb[b][lev[b]] + lb[b][lev[b] + 1] <= budget:
                    if best is None or h[b] > h[best]:
                        best = b
            if best is None:
                break
            total += lb[best][lev[best] + 1] - lb[best][lev[best]]
            lev[best] += 1
    else:
        while total > budget:
            best = None
            for b in range(len(h)):
                if lev[b] > 0 and (best is None or h[b] < h[best]):
                    best = b
            if best is None:
                break
            total += lb[best][lev[best] - 1] - lb[best][lev[best]]
            lev[best] -= 1
    return np.array(lev, dtype=np.int32), total, total <= budget
