"""Group-wise asymmetric round-to-nearest quantisation and bit packing (oracle).

Test infrastructure only.

The pages fix the target (low-bit integers after SINQ's dual-axis balancing:
[SINQ] 4-bit and, in some cases, 3-bit; EWQ's 8-bit middle tier) and that
groups are quantised independently ([BitNet] "Lượng Tử Hóa Nhóm và Chuẩn
Hóa").  They leave the affine details open; the reading used here:

* balanced values  x = W / (s t^T)  (s, t from the Sinkhorn step, or 1);
* a group is ``group`` consecutive columns of one row;
* lo = min(0, min x), hi = max(0, max x)  (the range always holds 0, so the
  integer zero-point lies in [0, 2^b - 1]);
* delta = (hi - lo) / (2^b - 1), z = rne(-lo / delta),
  q = clamp(rne(x / delta) + z, 0, 2^b - 1);  round half to even;
* a group with delta = 0 (or a delta whose reciprocal overflows) gets z = 0
  and q = 0;
* codes are packed as an LSB-first bit stream per row: the code of column j
  occupies bits [b*j, b*j + b) of the row's little-endian byte string;
* dequantisation: W' = s_i t_j (q - z) delta.

``quantize_groupwise_f32`` takes every rounding decision in fp32 with the
exact operation sequence the kernels use (reciprocals 1/s, 1/t and 1/delta,
each correctly rounded; products rounded once each), so its codes, deltas
and zero-points are bit-identical to a correct kernel's.
``quantize_groupwise_f64`` is the same definition with true fp64 divisions.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def _as_f32(w) -> np.ndarray:
    a = np.asarray(w)
    if a.dtype != np.float32:
        a = a.astype(np.float32)  # bf16 / fp32 inputs convert exactly
    return a


def balanced_f32(w, s=None, t=None) -> np.ndarray:
    """x_ij = (w_ij * (1/s_i)) * (1/t_j), each step one fp32 rounding."""
    x = _as_f32(w)
    if s is not None:
        rs = F32(1.0) / np.asarray(s, dtype=F32)
        x = x * rs[:, None]
    if t is not None:
        ct = F32(1.0) / np.asarray(t, dtype=F32)
        x = x * ct[None, :]
    return x


def _check_shape(rows: int, cols: int, bits: int, group: int):
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be one of 2, 3, 4, 8")
    if group <= 0 or cols % group:
        raise ValueError("group must divide cols")
    if (cols * bits) % 8:
        raise ValueError("cols*bits must be a whole number of bytes")


def quantize_groupwise_f32(w, s=None, t=None, bits: int = 4, group: int = 64):
    """Codes q (uint8 [rows, cols]), delta (f32 [rows, cols/group]), z (uint8)."""
    x = balanced_f32(w, s, t)
    rows, cols = x.shape
    _check_shape(rows, cols, bits, group)
    qmax = F32(2 ** bits - 1)
    xg = x.reshape(rows, cols // group, group)
    lo = np.minimum(F32(0), xg.min(axis=2))
    hi = np.maximum(F32(0), xg.max(axis=2))
    d = (hi - lo).astype(F32)
    delta = (d / qmax).astype(F32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        inv = (F32(1.0) / delta).astype(F32)
        ok = np.isfinite(inv)
        inv_s = np.where(ok, inv, F32(0))
        z = np.clip(np.rint((-lo) * inv_s), 0, qmax)
        q = np.clip(np.rint(xg * inv_s[:, :, None]) + z[:, :, None], 0, qmax)
    z = np.where(ok, z, 0)
    q = np.where(ok[:, :, None], q, 0)
    return (q.reshape(rows, cols).astype(np.uint8), delta.astype(F32),
            z.astype(np.uint8))


def quantize_groupwise_f64(w, s=None, t=None, bits: int = 4, group: int = 64):
    """Same definition with fp64 divisions: W / (s t^T), x / delta, -lo / delta."""
    x = np.asarray(w, dtype=np.float64)
    if s is not None:
        x = x / np.asarray(s, dtype=np.float64)[:, None]
    if t is not None:
        x = x / np.asarray(t, dtype=np.float64)[None, :]
    rows, cols = x.shape
    _check_shape(rows, cols, bits, group)
    qmax = float(2 ** bits - 1)
    xg = x.reshape(rows, cols // group, group)
    lo = np.minimum(0.0, xg.min(axis=2))
    hi = np.maximum(0.0, xg.max(axis=2))
    delta = (hi - lo) / qmax
    ok = delta > 0
    ds = np.where(ok, delta, 1.0)
    z = np.where(ok, np.clip(np.rint(-lo / ds), 0, qmax), 0)
    q = np.clip(np.rint(xg / ds[:, :, None]) + z[:, :, None], 0, qmax)
    q = np.where(ok[:, :, None], q, 0)
    return q.reshape(rows, cols).astype(np.uint8), delta, z.astype(np.uint8)


def near_tie_fraction(w, s, t, delta, z, bits: int, group: int, eps: float = 1e-5):
    """Mask of elements whose rounding is a near tie, in fp64 from given s, t, delta.

    An element is a near tie if u = x / delta has |u - floor(u) - 0.5| < eps;
    every element of a group whose zero-point argument -lo / delta is a near
    tie counts as well (the whole group may then shift by one code).
    """
    x = np.asarray(w, dtype=np.float64)
    if s is not None:
        x = x / np.asarray(s, dtype=np.float64)[:, None]
    if t is not None:
        x = x / np.asarray(t, dtype=np.float64)[None, :]
    rows, cols = x.shape
    xg = x.reshape(rows, cols // group, group)
    d = np.asarray(delta, dtype=np.float64)
    ds = np.where(d > 0, d, 1.0)
    u = xg / ds[:, :, None]
    tie = np.abs(u - np.floor(u) - 0.5) < eps
    lo = np.minimum(0.0, xg.min(axis=2))
    uz = -lo / ds
    ztie = np.abs(uz - np.floor(uz) - 0.5) < eps
    tie |= ztie[:, :, None]
    return tie.reshape(rows, cols)


def pack_codes(q, bits: int) -> np.ndarray:
    """LSB-first bit stream per row: uint8 [rows, cols*bits/8]."""
    q = np.asarray(q, dtype=np.uint16)
    rows, cols = q.shape
    if (cols * bits) % 8:
        raise ValueError("cols*bits must be a whole number of bytes")
    planes = ((q[:, :, None] >> np.arange(bits, dtype=np.uint16)) & 1).astype(np.uint8)
    return np.packbits(planes.reshape(rows, cols * bits), axis=1, bitorder="little")


def unpack_codes(packed, bits: int, cols: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    planes = np.unpackbits(packed, axis=1, bitorder="little")[:, : cols * bits]
    planes = planes.reshape(rows, cols, bits).astype(np.uint16)
    return np.sum(planes << np.arange(bits, dtype=np.uint16), axis=2).astype(np.uint8)


def dequantize_f32(q, delta, z, s=None, t=None, group: int = 64) -> np.ndarray:
    """W' = ((q - z) * delta) * s_i * t_j in fp32, one rounding per product."""
    q = np.asarray(q)
    rows, cols = q.shape
    d = np.repeat(np.asarray(delta, dtype=F32), group, axis=1)
    zz = np.repeat(np.asarray(z, dtype=np.int32), group, axis=1)
    y = (q.astype(np.int32) - zz).astype(F32) * d
    if s is not None:
        y = y * np.asarray(s, dtype=F32)[:, None]
    if t is not None:
        y = y * np.asarray(t, dtype=F32)[None, :]
    return y.astype(F32)
