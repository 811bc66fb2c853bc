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
each correctly rounded; products rounded once each; the zero-point ratio and
any element ratio near a half-way point by one correctly rounded division),
so its codes, deltas and zero-points are bit-identical to a correct
kernel's.
``quantize_groupwise_f64`` is the plain definition with true fp64 divisions
(the reference for the spec code bar: codes bit-exact except near
ties, see ``near_tie_mask``).
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


# A fast ratio u = x * (1/delta) is within a few fp32 ulps of the exact ratio
# (2^b - 1) * x / (hi - lo): at most about 6.1e-5 away for 8-bit codes.  When
# u lies within NEAR_HALF of a half-way point the ratio is recomputed with one
# correctly rounded division, which returns exactly k + 1/2 whenever the exact
# ratio is k + 1/2 and its operands are exact (bf16 / fp32 inputs without
# scales).
NEAR_HALF = F32(0.5 - 2.0 ** -13)


def quantize_groupwise_f32(w, s=None, t=None, bits: int = 4, group: int = 64):
    """Codes q (uint8 [rows, cols]), delta (f32 [rows, cols/group]), z (uint8).

    The fp32 decision sequence (every step one correctly rounded fp32
    operation): x = (w * (1/s_i)) * (1/t_j); per group lo = min(0, min x),
    hi = max(0, max x), d = hi - lo, delta = d / (2^b - 1), inv = 1 / delta;
    a group whose inv is not finite gets z = 0 and q = 0; otherwise
    z = clamp(rne(uz)) with uz = -lo * inv, or uz = ((2^b - 1) * -lo) / d when
    |uz - rne(uz)| > NEAR_HALF; per element u = x * inv, and when the
    matrix has no scales or b = 8 (where ratios can be exact half-way points,
    or the fast ratio's error can exceed the 1e-5 near-tie window) u =
    ((2^b - 1) * x) / d when |u - rne(u)| > NEAR_HALF; then
    q = clamp(rne(u) + z, 0, 2^b - 1)."""
    x = balanced_f32(w, s, t)
    rows, cols = x.shape
    _check_shape(rows, cols, bits, group)
    qmax = F32(2 ** bits - 1)
    exact = (s is None and t is None) or bits == 8
    xg = x.reshape(rows, cols // group, group)
    lo = np.minimum(F32(0), xg.min(axis=2))
    hi = np.maximum(F32(0), xg.max(axis=2))
    d = (hi - lo).astype(F32)
    delta = (d / qmax).astype(F32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        inv = (F32(1.0) / delta).astype(F32)
        ok = np.isfinite(inv)
        inv_s = np.where(ok, inv, F32(0))
        ds = np.where(ok & (d > 0), d, F32(1))
        uz = (-lo) * inv_s
        rz = np.rint(uz)
        rz = np.where(np.abs(uz - rz) > NEAR_HALF, np.rint((qmax * -lo) / ds), rz)
        z = np.clip(rz, 0, qmax)
        u = xg * inv_s[:, :, None]
        r = np.rint(u)
        if exact:
            near = np.abs(u - r) > NEAR_HALF
            r = np.where(near, np.rint((qmax * xg) / ds[:, :, None]), r)
        q = np.clip(r + z[:, :, None], 0, qmax)
    z = np.where(ok, z, 0)
    q = np.where(ok[:, :, None], q, 0)
    return (q.reshape(rows, cols).astype(np.uint8), delta.astype(F32),
            z.astype(np.uint8))


def balanced_f64(w, s=None, t=None) -> np.ndarray:
    """x_ij = w_ij / (s_i t_j) in fp64 (true divisions)."""
    x = np.asarray(w, dtype=np.float64)
    if s is not None:
        x = x / np.asarray(s, dtype=np.float64)[:, None]
    if t is not None:
        x = x / np.asarray(t, dtype=np.float64)[None, :]
    return x


def _group_ratios_f64(x, bits: int, group: int):
    """Per group: span = hi - lo, the zero-point argument -lo / delta and every
    element's x / delta, in fp64.  Since delta = span / (2^b - 1), the ratios
    are evaluated as (2^b - 1) * value / span: the numerator and the span are
    exact in fp64 for bf16 / fp32 inputs without scales, so a ratio whose exact
    value is a half-way point k + 1/2 comes out as exactly k + 1/2 and is
    rounded as the definition says (half to even).  Returns (lo, span, uz, u)
    with uz and u set to 0 where span = 0."""
    rows, cols = x.shape
    _check_shape(rows, cols, bits, group)
    qmax = float(2 ** bits - 1)
    xg = x.reshape(rows, cols // group, group)
    lo = np.minimum(0.0, xg.min(axis=2))
    hi = np.maximum(0.0, xg.max(axis=2))
    span = hi - lo
    ok = span > 0
    sp = np.where(ok, span, 1.0)
    uz = np.where(ok, (qmax * -lo) / sp, 0.0)
    u = np.where(ok[:, :, None], (qmax * xg) / sp[:, :, None], 0.0)
    return lo, span, uz, u


def quantize_groupwise_f64(w, s=None, t=None, bits: int = 4, group: int = 64):
    """The plain definition in fp64: x = W / (s t^T) with true divisions,
    delta = (hi - lo) / (2^b - 1), z = clamp(rne(-lo / delta)), q = clamp(rne(x /
    delta) + z); the two ratios are evaluated without rounding delta first
    (``_group_ratios_f64``).  Returns q (uint8), delta (fp64), z (uint8)."""
    x = balanced_f64(w, s, t)
    rows, cols = x.shape
    qmax = float(2 ** bits - 1)
    lo, span, uz, u = _group_ratios_f64(x, bits, group)
    ok = span > 0
    z = np.where(ok, np.clip(np.rint(uz), 0, qmax), 0)
    q = np.clip(np.rint(u) + z[:, :, None], 0, qmax)
    q = np.where(ok[:, :, None], q, 0)
    return q.reshape(rows, cols).astype(np.uint8), span / qmax, z.astype(np.uint8)


def near_tie_mask(w, s, t, bits: int, group: int, eps: float = 1e-5) -> np.ndarray:
    """Elements whose code the definition decides within ``eps`` of a rounding
    boundary, from the plain fp64 definition with the given s and t.

    An element is a near tie if its ratio u = x / delta has
    |u - floor(u) - 0.5| < eps.  When the zero-point's ratio -lo / delta is a
    near tie, the whole group may shift by one code, so every element of that
    group counts as well.  bool [rows, cols].
    """
    x = balanced_f64(w, s, t)
    rows, cols = x.shape
    _, span, uz, u = _group_ratios_f64(x, bits, group)

    def near(v):
        return np.abs(v - np.floor(v) - 0.5) < eps

    ok = (span > 0)[:, :, None]
    tie = ok & (near(u) | near(uz)[:, :, None])
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
