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
