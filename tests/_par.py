"""Helpers for running the CPU oracle over many matrices in the GPU tests.

The oracle's work is numpy array kernels, which release the GIL, so a thread
pool runs it on all host cores without starting processes from a program
that has initialised the GPU.  Workers: the host cores this process may use,
at most 16 (one GPU's share of a machine's cores)."""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def pmap(fn, items):
    items = list(items)
    with cf.ThreadPoolExecutor(workers()) as ex:
        return list(ex.map(fn, items))


def host_f32(t: torch.Tensor) -> np.ndarray:
    """A device matrix as host fp32 (bf16 widened exactly, in numpy)."""
    if t.dtype == torch.bfloat16:
        u = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return (u.astype(np.uint32) << 16).view(np.float32)
    return t.contiguous().cpu().numpy().astype(np.float32, copy=False)
