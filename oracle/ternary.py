"""Ternary {-1, 0, +1} weights with a per-row scale (oracle).  Test infrastructure only.

[BitNet] "Hệ Thống Trọng Số Ternary": each parameter takes one of the three
values -1, 0, +1 (about 1.58 bits); EWQ ([EWQ] step 2) names 1.58-bit as the
aggressive option for its lowest-entropy blocks.  The page's own weight
formula, Sign(W - alpha) with alpha the mean, yields only +-1, and its
BitLinear scale beta is described only as a factor that reduces the
approximation error.  Reading used here, the plainest closed form that keeps
the three values and a per-row scale: beta_i = mean_j |W_ij| (no centring),
q = clamp(rne(W_ij / beta_i), -1, 1), stored as the 2-bit code q + 1, LSB-first
as in ``rtn.pack_codes``.  A row with beta = 0 gets q = 0.

``ternary_quantize`` stores beta as fp32 (the mean in fp64, rounded once)
and takes the code decision in fp32 as w * (1/beta) with the reciprocal
correctly rounded, the operation sequence of the kernels, so its codes
compare bit for bit.  ``ternary_quantize_f64`` is the plain definition in
fp64 (beta not rounded, true division w / beta), the reference for the code
bar: codes equal except near ties (``ternary_near_tie_mask``).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def ternary_quantize(w, beta=None):
    """Return (q in {-1,0,1} int8 [rows, cols], beta fp32 [rows]).

    ``beta`` may be given (stage isolation: decide codes from another
    implementation's scale); otherwise it is mean |W| per row.
    """
    a = np.asarray(w)
    if beta is None:
        beta = np.mean(np.abs(a.astype(np.float64)), axis=1).astype(F32)
    beta = np.asarray(beta, dtype=F32)
    x = a.astype(F32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        inv = (F32(1.0) / beta).astype(F32)
        ok = np.isfinite(inv)
        q = np.clip(np.rint(x * np.where(ok, inv, F32(0))[:, None]), -1, 1)
    q = np.where(ok[:, None], q, 0)
    return q.astype(np.int8), beta


def ternary_dequantize(q, beta) -> np.ndarray:
    return (np.asarray(q, dtype=F32) * np.asarray(beta, dtype=F32)[:, None]).astype(F32)


def ternary_quantize_f64(w):
    """The plain definition in fp64: beta_i = mean_j |W_ij| (not rounded),
    q = clamp(rne(W_ij / beta_i), -1, 1), q = 0 on a row with beta = 0.
    Returns (q int8 [rows, cols], beta fp64 [rows])."""
    a = np.asarray(w, dtype=np.float64)
    beta = np.mean(np.abs(a), axis=1)
    ok = beta > 0
    b = np.where(ok, beta, 1.0)
    q = np.clip(np.rint(a / b[:, None]), -1, 1)
    q = np.where(ok[:, None], q, 0)
    return q.astype(np.int8), beta


def ternary_near_tie_mask(w, beta=None, eps: float = 1e-5) -> np.ndarray:
    """Elements whose ternary code the definition decides within ``eps`` of a
    rounding boundary: u = |W_ij| / beta_i (fp64; beta the fp64 row mean unless
    given) with |u - floor(u) - 0.5| < eps.  Only u near 1/2 can change the
    code (rounding at 3/2 and above is clipped to 1 either way), but every
    half-way point is flagged, as for the affine grid.  bool [rows, cols]."""
    a = np.abs(np.asarray(w, dtype=np.float64))
    if beta is None:
        beta = np.mean(a, axis=1)
    beta = np.asarray(beta, dtype=np.float64)
    ok = beta > 0
    u = a / np.where(ok, beta, 1.0)[:, None]
    return ok[:, None] & (np.abs(u - np.floor(u) - 0.5) < eps)
