"""MI355X-native calibration-free weight-quantisation pass.

Python binding over libwoq.so (hand-written HIP kernels for gfx950 behind the
C ABI of include/woq.h).  Each function has the name of the C entry point it
wraps and does argument marshalling only: torch tensors provide device memory
and the current HIP stream; every step of the pass runs in the library's
kernels.  There is no CPU or PyTorch fallback: if libwoq.so is missing the
calls raise.  Since the library takes raw pointers, the binding first checks
that every tensor is on one GPU and that caller-supplied buffers come one per
matrix, with the right dtype and at least the size the call reads or writes
(ValueError / TypeError before anything is enqueued).  Input matrices may be
row-strided views (unit column stride, row stride >= cols, for example a
column slice of a fused projection weight); they are passed with their row
stride.  Workspaces and outputs the binding allocates are allocated on the
stream the call runs on, so the caching allocator never hands their memory
to another stream while the call's kernels may still use it.

  ewq_block_entropy     EWQ per-matrix softmax entropy, block entropy, tiers
  sinq_balance          SINQ dual-axis Sinkhorn std balancing -> (s, t)
  quant_pack_groupwise  group-wise asymmetric RTN with LSB-first bit packing
  dequant_unpack        inverse map (codes -> weights)
  ternary_pack          ternary {-1, 0, +1} codes with a per-row scale
  ewq_budget_levels     EWQ's budgeted placement: precision levels to a budget
                        (host-side)
  df11_*                lossless exponent code for the blocks kept in bf16:
                        df11_exponent_histogram, df11_build_code (host),
                        df11_buffer_sizes (host), df11_encode, df11_decode;
                        df11_compress chains the first three steps
"""
from __future__ import annotations

import contextlib
import ctypes
from typing import List, Optional, Sequence

import torch

from . import _lib
from ._lib import WoqError  # noqa: F401

__all__ = ["ewq_block_entropy", "sinq_balance", "quant_pack_groupwise",
           "dequant_unpack", "ternary_pack", "ewq_budget_levels", "workspace_size", "WoqError",
           "df11_buffer_sizes", "df11_exponent_histogram", "df11_build_code", "df11_encode",
           "df11_decode", "df11_compress", "codebook_normal", "quant_pack_codebook",
           "dequant_codebook", "nonfinite_count"]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _lib.WOQ_BF16
    if t.dtype == torch.float32:
        return _lib.WOQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ld(t: torch.Tensor) -> int:
    """Row stride passed to the library: 0 for a contiguous matrix, else the
    tensor's row stride (the library checks its rules)."""
    return 0 if t.is_contiguous() else int(t.stride(0))


def _descs(tensors: Sequence[torch.Tensor]) -> List[tuple]:
    """Checks the matrices and returns their (data_ptr, dtype code, rows,
    cols, ld) descriptors (one pass over the list)."""
    if len(tensors) == 0:
        raise ValueError("at least one matrix is required")
    out = []
    for t in tensors:
        if t.dim() != 2:
            raise ValueError("matrices must be 2-D")
        r, c = t.shape
        if r < 1 or c < 1:
            raise ValueError(f"empty matrix of shape {tuple(t.shape)}")
        ld = 0
        if not t.is_contiguous():
            s0, s1 = t.stride()
            if s1 != 1 or s0 < c:
                raise ValueError("matrices must be contiguous or row-strided views "
                                 f"(unit column stride), got strides {(s0, s1)}")
            ld = s0
        out.append((t.data_ptr(), _dtype_code(t), r, c, ld))
    return out


def _check_mats(tensors: Sequence[torch.Tensor]) -> None:
    _descs(tensors)


def _mats(tensors: Sequence[torch.Tensor]):
    return _lib.mat_array(_descs(tensors))


def _check_bufs(name: str, ts, sizes, dtype) -> None:
    """Caller-supplied per-matrix buffers: one per matrix, of the dtype,
    contiguous and large enough, since the library reads or writes that many
    elements through the raw pointer.  None (the whole list or an entry) is
    left to the library's own NULL checks."""
    if ts is None:
        return
    if len(ts) != len(sizes):
        raise ValueError(f"{name}: {len(ts)} tensors for {len(sizes)} matrices")
    for i, (t, n) in enumerate(zip(ts, sizes)):
        if t is None:
            continue
        if t.dtype != dtype:
            raise TypeError(f"{name}[{i}]: dtype {t.dtype}, expected {dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name}[{i}] must be contiguous")
        if t.numel() < n:
            raise ValueError(f"{name}[{i}] holds {t.numel()} elements, {n} needed")


def _device(*groups):
    """The one GPU every given tensor lives on (the library takes raw device
    pointers, so a host tensor must never reach it)."""
    dev = None
    for g in groups:
        if g is None:
            continue
        for t in (g if isinstance(g, (list, tuple)) else [g]):
            if t is None:
                continue
            if t.device.type != "cuda":
                raise ValueError(f"tensors must be on a GPU, got one on {t.device}")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"tensors on two devices: {dev} and {t.device}")
    if dev is None:
        raise ValueError("no GPU tensor given")
    return dev


def _group_cols(m: torch.Tensor, group: int) -> int:
    return group if group > 0 else m.shape[1]


def _stream(stream, device=None) -> Optional[int]:
    """The HIP stream handle: the given stream, else the current stream of the
    tensors' device."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _on(stream, device):
    """Context for the binding's own allocations: the call's stream when one is
    given (a torch stream or a raw handle), so that the caching allocator
    keeps the memory for that stream; otherwise the current stream."""
    if stream is None:
        return contextlib.nullcontext()
    if not isinstance(stream, torch.cuda.Stream):
        stream = torch.cuda.ExternalStream(int(stream), device=device)
    return torch.cuda.stream(stream)


def nonfinite_count(ws: torch.Tensor) -> torch.Tensor:
    """The non-finite weight count that ewq_block_entropy and sinq_balance
    write into the head of their workspace: an int64 view of ws[0:8]."""
    return ws[:8].view(torch.int64)


def _ptrs(ts):
    if ts is None:
        return None
    return _lib.ptr_array(None if t is None else t.data_ptr() for t in ts)


def workspace_size(op: int, mats: Sequence[torch.Tensor], group: int = 0) -> int:
    lib = _lib.load()
    arr = _mats(mats)
    out = ctypes.c_size_t(0)
    _lib.check("woq_workspace_size", lib.woq_workspace_size(op, arr, len(mats), group,
                                                             ctypes.byref(out)))
    return out.value


def _workspace(op, mats, group, ws, device):
    """The caller's workspace, or a new one on the current stream (callers
    allocate inside ``_on``)."""
    if ws is not None and ws.dtype != torch.uint8:
        raise TypeError(f"workspace must be uint8 (bytes), got {ws.dtype}")
    if ws is not None and not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    need = workspace_size(op, mats, group)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, _lib.WS_HEAD), dtype=torch.uint8, device=device)
    return ws


def ewq_block_entropy(mats: Sequence[torch.Tensor], block_id: Optional[Sequence[int]] = None,
                      n_blocks: int = 1, x: float = 1.0, *, exp_hist=None, ws=None, stream=None):
    """Per-matrix entropy, block entropy, (mu, sigma, T), tiers and order (device
    tensors), and the count of NaN / inf weights (``nonfinite``, a view of the
    workspace head).  ``exp_hist``: True, or an int32 device tensor of
    n_mats * 256 elements, to also get each bf16 matrix's exponent histogram
    from the same pass (ewq_block_entropy_ex); returned as ``exp_hist``
    [n_mats, 256]."""
    lib = _lib.load()
    _check_mats(mats)
    n = len(mats)
    if block_id is not None and len(block_id) != n:
        raise ValueError(f"block_id: {len(block_id)} ids for {n} matrices")
    eh = exp_hist if isinstance(exp_hist, torch.Tensor) else None
    if eh is not None:
        _check_bufs("exp_hist", [eh], [256 * n], torch.int32)
    dev = _device(mats, ws, eh)
    arr = _mats(mats)
    with _on(stream, dev):
        h_mat = torch.empty(n, dtype=torch.float64, device=dev)
        h_block = torch.empty(n_blocks, dtype=torch.float64, device=dev)
        stats = torch.empty(3, dtype=torch.float64, device=dev)
        tier = torch.empty(n_blocks, dtype=torch.int32, device=dev)
        order = torch.empty(n_blocks, dtype=torch.int32, device=dev)
        if exp_hist is True:
            eh = torch.empty(n, 256, dtype=torch.int32, device=dev)
        ws = _workspace(_lib.OP_ENTROPY, mats, 0, ws, dev)
    bid = None
    if block_id is not None:
        bid = (ctypes.c_int32 * n)(*[int(b) for b in block_id])
    ptrs = (h_mat.data_ptr(), h_block.data_ptr(), stats.data_ptr(), tier.data_ptr(),
            order.data_ptr())
    if eh is None:
        st = lib.ewq_block_entropy(arr, n, bid, n_blocks, float(x), *ptrs, ws.data_ptr(),
                                   ws.numel(), _stream(stream, dev))
        _lib.check("ewq_block_entropy", st)
    else:
        st = lib.ewq_block_entropy_ex(arr, n, bid, n_blocks, float(x), *ptrs, eh.data_ptr(),
                                      ws.data_ptr(), ws.numel(), _stream(stream, dev))
        _lib.check("ewq_block_entropy_ex", st)
    out = {"h_mat": h_mat, "h_block": h_block, "stats": stats, "tier": tier, "order": order,
           "nonfinite": nonfinite_count(ws)}
    if eh is not None:
        out["exp_hist"] = eh.view(n, 256)
    return out


def sinq_balance(mats: Sequence[torch.Tensor], iters: int, *, rms: bool = False,
                 shared: bool = False, row_scale=None, col_scale=None, ws=None, stream=None):
    """Row scales s [rows] and column scales t [cols] (fp32) per matrix.
    ``rms``: root mean square in place of the centred std; ``shared``: the
    call runs beside another on the same GPU, strips planned for half of it
    (both through sinq_balance_ex)."""
    lib = _lib.load()
    _check_mats(mats)
    _check_bufs("row_scale", row_scale, [m.shape[0] for m in mats], torch.float32)
    _check_bufs("col_scale", col_scale, [m.shape[1] for m in mats], torch.float32)
    dev = _device(mats, row_scale, col_scale, ws)
    arr = _mats(mats)
    with _on(stream, dev):
        if row_scale is None:
            row_scale = [torch.empty(m.shape[0], dtype=torch.float32, device=dev) for m in mats]
        if col_scale is None:
            col_scale = [torch.empty(m.shape[1], dtype=torch.float32, device=dev) for m in mats]
        ws = _workspace(_lib.OP_SINQ, mats, 0, ws, dev)
    flags = (_lib.WOQ_SINQ_RMS if rms else 0) | (_lib.WOQ_SINQ_SHARED if shared else 0)
    if flags:
        st = lib.sinq_balance_ex(arr, len(mats), int(iters), flags, _ptrs(row_scale),
                                 _ptrs(col_scale), ws.data_ptr(), ws.numel(), _stream(stream, dev))
        _lib.check("sinq_balance_ex", st)
    else:
        st = lib.sinq_balance(arr, len(mats), int(iters), _ptrs(row_scale), _ptrs(col_scale),
                              ws.data_ptr(), ws.numel(), _stream(stream, dev))
        _lib.check("sinq_balance", st)
    return row_scale, col_scale


def quant_pack_groupwise(mats: Sequence[torch.Tensor], bits: int, group: int, *,
                         row_scale=None, col_scale=None, codes=None, scales=None, zeros=None,
                         ws=None, stream=None):
    """Packed codes (uint8 [rows, cols*bits/8]), deltas (fp32) and zero-points (uint8)."""
    lib = _lib.load()
    _check_mats(mats)

    def g(m):
        return _group_cols(m, group)
    _check_bufs("row_scale", row_scale, [m.shape[0] for m in mats], torch.float32)
    _check_bufs("col_scale", col_scale, [m.shape[1] for m in mats], torch.float32)
    _check_bufs("codes", codes, [m.shape[0] * (m.shape[1] * bits // 8) for m in mats], torch.uint8)
    _check_bufs("scales", scales, [m.shape[0] * (m.shape[1] // g(m)) for m in mats], torch.float32)
    _check_bufs("zeros", zeros, [m.shape[0] * (m.shape[1] // g(m)) for m in mats], torch.uint8)
    dev = _device(mats, row_scale, col_scale, codes, scales, zeros, ws)
    arr = _mats(mats)
    with _on(stream, dev):
        if codes is None:
            codes = [torch.empty(m.shape[0], m.shape[1] * bits // 8, dtype=torch.uint8, device=dev)
                     for m in mats]
        if scales is None:
            scales = [torch.empty(m.shape[0], m.shape[1] // g(m), dtype=torch.float32, device=dev)
                      for m in mats]
        if zeros is None:
            zeros = [torch.empty(m.shape[0], m.shape[1] // g(m), dtype=torch.uint8, device=dev)
                     for m in mats]
        ws = _workspace(_lib.OP_QUANT, mats, group, ws, dev)
    st = lib.quant_pack_groupwise(arr, len(mats), _ptrs(row_scale), _ptrs(col_scale), int(bits),
                                  int(group), _ptrs(codes), _ptrs(scales), _ptrs(zeros),
                                  ws.data_ptr(), ws.numel(), _stream(stream, dev))
    _lib.check("quant_pack_groupwise", st)
    return codes, scales, zeros


def dequant_unpack(shapes, codes, scales, bits: int, group: int, *, zeros=None, row_scale=None,
                   col_scale=None, out_dtype=torch.float32, out=None, ws=None, stream=None):
    """Decode packed codes back to weights W' = (((q - z) delta) s_i) t_j."""
    lib = _lib.load()
    shapes = [(int(r), int(c)) for (r, c) in shapes]
    if len(shapes) == 0 or min(min(rc) for rc in shapes) < 1:
        raise ValueError("at least one matrix is required, none of them empty")

    def g(rc):
        return group if group > 0 else rc[1]
    _check_bufs("codes", codes, [r * (c * bits // 8) for r, c in shapes], torch.uint8)
    _check_bufs("scales", scales, [r * (c // g((r, c))) for r, c in shapes], torch.float32)
    _check_bufs("zeros", zeros, [r * (c // g((r, c))) for r, c in shapes], torch.uint8)
    _check_bufs("row_scale", row_scale, [r for r, _ in shapes], torch.float32)
    _check_bufs("col_scale", col_scale, [c for _, c in shapes], torch.float32)
    if out is not None and [tuple(o.shape) for o in out] != shapes:
        raise ValueError("out: tensors do not have the given shapes")
    dev = _device(codes, scales, zeros, row_scale, col_scale, out, ws)
    with _on(stream, dev):
        if out is None:
            out = [torch.empty(r, c, dtype=out_dtype, device=dev) for (r, c) in shapes]
        arr = _mats(out)
        ws = _workspace(_lib.OP_DEQUANT, out, group, ws, dev)
    st = lib.dequant_unpack(arr, len(out), _ptrs(codes), _ptrs(scales), _ptrs(zeros),
                            _ptrs(row_scale), _ptrs(col_scale), int(bits), int(group),
                            ws.data_ptr(), ws.numel(), _stream(stream, dev))
    _lib.check("dequant_unpack", st)
    return out


def codebook_normal(bits: int) -> list:
    """The normal-quantile code book of 2^bits fp32 levels (ascending, largest 1)."""
    lib = _lib.load()
    buf = (ctypes.c_float * (1 << int(bits)))()
    _lib.check("woq_codebook_normal", lib.woq_codebook_normal(int(bits), buf))
    return list(buf)


def _levels(bits: int, levels):
    """Host fp32 array of the code book (default: the normal-quantile book)."""
    lv = codebook_normal(bits) if levels is None else [float(v) for v in levels]
    if len(lv) != 1 << int(bits):
        raise ValueError(f"a {bits}-bit code book has {1 << int(bits)} levels, got {len(lv)}")
    return (ctypes.c_float * len(lv))(*lv)


def quant_pack_codebook(mats: Sequence[torch.Tensor], bits: int, group: int, *, levels=None,
                        row_scale=None, col_scale=None, codes=None, scales=None, ws=None,
                        stream=None):
    """Packed codes (uint8 [rows, cols*bits/8]) of the nearest code-book level and the
    per-group scales a = max |x| (fp32); levels default to the normal-quantile book."""
    lib = _lib.load()
    _check_mats(mats)
    lv = _levels(bits, levels)

    def g(m):
        return _group_cols(m, group)
    _check_bufs("row_scale", row_scale, [m.shape[0] for m in mats], torch.float32)
    _check_bufs("col_scale", col_scale, [m.shape[1] for m in mats], torch.float32)
    _check_bufs("codes", codes, [m.shape[0] * (m.shape[1] * bits // 8) for m in mats], torch.uint8)
    _check_bufs("scales", scales, [m.shape[0] * (m.shape[1] // g(m)) for m in mats], torch.float32)
    dev = _device(mats, row_scale, col_scale, codes, scales, ws)
    arr = _mats(mats)
    with _on(stream, dev):
        if codes is None:
            codes = [torch.empty(m.shape[0], m.shape[1] * bits // 8, dtype=torch.uint8, device=dev)
                     for m in mats]
        if scales is None:
            scales = [torch.empty(m.shape[0], m.shape[1] // g(m), dtype=torch.float32, device=dev)
                      for m in mats]
        ws = _workspace(_lib.OP_QUANT, mats, group, ws, dev)
    st = lib.quant_pack_codebook(arr, len(mats), _ptrs(row_scale), _ptrs(col_scale), int(bits),
                                 int(group), lv, _ptrs(codes), _ptrs(scales), ws.data_ptr(),
                                 ws.numel(), _stream(stream, dev))
    _lib.check("quant_pack_codebook", st)
    return codes, scales


def dequant_codebook(shapes, codes, scales, bits: int, group: int, *, levels=None, row_scale=None,
                     col_scale=None, out_dtype=torch.float32, out=None, ws=None, stream=None):
    """Decode code-book codes back to weights W' = ((a l_q) s_i) t_j."""
    lib = _lib.load()
    lv = _levels(bits, levels)
    shapes = [(int(r), int(c)) for (r, c) in shapes]
    if len(shapes) == 0 or min(min(rc) for rc in shapes) < 1:
        raise ValueError("at least one matrix is required, none of them empty")

    def g(rc):
        return group if group > 0 else rc[1]
    _check_bufs("codes", codes, [r * (c * bits // 8) for r, c in shapes], torch.uint8)
    _check_bufs("scales", scales, [r * (c // g((r, c))) for r, c in shapes], torch.float32)
    _check_bufs("row_scale", row_scale, [r for r, _ in shapes], torch.float32)
    _check_bufs("col_scale", col_scale, [c for _, c in shapes], torch.float32)
    if out is not None and [tuple(o.shape) for o in out] != shapes:
        raise ValueError("out: tensors do not have the given shapes")
    dev = _device(codes, scales, row_scale, col_scale, out, ws)
    with _on(stream, dev):
        if out is None:
            out = [torch.empty(r, c, dtype=out_dtype, device=dev) for (r, c) in shapes]
        arr = _mats(out)
        ws = _workspace(_lib.OP_DEQUANT, out, group, ws, dev)
    st = lib.dequant_codebook(arr, len(out), _ptrs(codes), _ptrs(scales), _ptrs(row_scale),
                              _ptrs(col_scale), int(bits), int(group), lv, ws.data_ptr(),
                              ws.numel(), _stream(stream, dev))
    _lib.check("dequant_codebook", st)
    return out


def ternary_pack(mats: Sequence[torch.Tensor], *, codes=None, row_scale=None, ws=None,
                 stream=None):
    """2-bit ternary codes (q + 1) and per-row beta."""
    lib = _lib.load()
    _check_mats(mats)
    _check_bufs("codes", codes, [m.shape[0] * (m.shape[1] // 4) for m in mats], torch.uint8)
    _check_bufs("row_scale", row_scale, [m.shape[0] for m in mats], torch.float32)
    dev = _device(mats, codes, row_scale, ws)
    arr = _mats(mats)
    with _on(stream, dev):
        if codes is None:
            codes = [torch.empty(m.shape[0], m.shape[1] // 4, dtype=torch.uint8, device=dev)
                     for m in mats]
        if row_scale is None:
            row_scale = [torch.empty(m.shape[0], dtype=torch.float32, device=dev) for m in mats]
        ws = _workspace(_lib.OP_TERNARY, mats, 0, ws, dev)
    st = lib.ternary_pack(arr, len(mats), _ptrs(codes), _ptrs(row_scale), ws.data_ptr(),
                          ws.numel(), _stream(stream, dev))
    _lib.check("ternary_pack", st)
    return codes, row_scale


def ewq_budget_levels(h_block: Sequence[float], level_bytes, level0: Sequence[int], budget: int):
    """Levels adjusted to a storage budget: (levels list, total bytes, fits).

    ``level_bytes[b][l]`` is block b's storage at level l (ascending)."""
    lib = _lib.load()
    n = len(h_block)
    nl = len(level_bytes[0]) if n else 0
    hb = (ctypes.c_double * n)(*[float(v) for v in h_block])
    lb = (ctypes.c_int64 * (n * nl))(*[int(x) for row in level_bytes for x in row])
    l0 = (ctypes.c_int32 * n)(*[int(v) for v in level0])
    out = (ctypes.c_int32 * n)()
    total = ctypes.c_int64(0)
    fits = ctypes.c_int32(0)
    _lib.check("ewq_budget_levels", lib.ewq_budget_levels(hb, lb, n, nl, l0, int(budget), out,
                                                          ctypes.byref(total), ctypes.byref(fits)))
    return list(out), total.value, bool(fits.value)


# ------------------------------------------------------------------ DF11
def df11_buffer_sizes(n: int, total_bits: int):
    """(n_seg, enc_bytes, gap_bytes, n_blocks) of an encoded matrix (host-side)."""
    lib = _lib.load()
    out = [ctypes.c_int64(0) for _ in range(4)]
    _lib.check("df11_buffer_sizes", lib.df11_buffer_sizes(int(n), int(total_bits),
                                                          *[ctypes.byref(o) for o in out]))
    return tuple(o.value for o in out)


def df11_exponent_histogram(mats: Sequence[torch.Tensor], *, hist=None, ws=None, stream=None):
    """Exponent counts per matrix: int32 tensor [n_mats, 256] on the device."""
    lib = _lib.load()
    _check_mats(mats)
    if hist is not None:
        _check_bufs("hist", [hist], [256 * len(mats)], torch.int32)
    dev = _device(mats, hist, ws)
    arr = _mats(mats)
    with _on(stream, dev):
        if hist is None:
            hist = torch.empty(len(mats), 256, dtype=torch.int32, device=dev)
        ws = _workspace(_lib.OP_DF11_HIST, mats, 0, ws, dev)
    st = lib.df11_exponent_histogram(arr, len(mats), hist.data_ptr(), ws.data_ptr(), ws.numel(),
                                     _stream(stream, dev))
    _lib.check("df11_exponent_histogram", st)
    return hist


def df11_build_code(hist):
    """The code of one exponent histogram (host-side): dict with code_len
    (uint8[256]), codeword (uint32[256]), tables (uint8[n_tables, 256]),
    total_bits."""
    import numpy as np
    lib = _lib.load()
    h = np.ascontiguousarray(np.asarray(hist, dtype=np.int64).reshape(256))
    code_len = np.zeros(256, dtype=np.uint8)
    codeword = np.zeros(256, dtype=np.uint32)
    tables = np.zeros(17 * 256, dtype=np.uint8)
    n_tables = ctypes.c_int32(0)
    total = ctypes.c_int64(0)
    st = lib.df11_build_code(h.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), code_len.ctypes.data,
                             codeword.ctypes.data, tables.ctypes.data, ctypes.byref(n_tables),
                             ctypes.byref(total))
    _lib.check("df11_build_code", st)
    return {"code_len": code_len, "codeword": codeword,
            "tables": tables[:256 * n_tables.value].reshape(n_tables.value, 256),
            "total_bits": total.value}


def _host_ptrs(arrays):
    arr = (ctypes.c_void_p * len(arrays))()
    for i, a in enumerate(arrays):
        arr[i] = a.ctypes.data
    return ctypes.cast(arr, _lib.PP)


def df11_encode(mats: Sequence[torch.Tensor], codes, *, ws=None, stream=None):
    """Encode each bf16 matrix with its code (one df11_build_code dict per
    matrix).  Returns one dict per matrix with the device buffers (enc, sm,
    gaps, block_pos, tables, code_len) and n_tables, total_bits, shape."""
    import numpy as np
    lib = _lib.load()
    _check_mats(mats)
    if len(codes) != len(mats):
        raise ValueError(f"codes: {len(codes)} codes for {len(mats)} matrices")
    dev = _device(mats, ws)
    arr = _mats(mats)
    # every matrix's tables and code lengths in one host-to-device copy
    host = np.concatenate([np.concatenate([np.ascontiguousarray(c["tables"], dtype=np.uint8).reshape(-1),
                                           np.ascontiguousarray(c["code_len"], dtype=np.uint8)])
                           for c in codes])
    outs, off = [], 0
    with _on(stream, dev):
        meta = torch.from_numpy(host).to(dev)
        for m, c in zip(mats, codes):
            _, eb, gb, nb = df11_buffer_sizes(m.numel(), c["total_bits"])
            nt = int(c["tables"].shape[0])
            outs.append({
                "enc": torch.empty(eb, dtype=torch.uint8, device=dev),
                "sm": torch.empty(m.numel(), dtype=torch.uint8, device=dev),
                "gaps": torch.empty(gb, dtype=torch.uint8, device=dev),
                "block_pos": torch.empty(nb + 1, dtype=torch.int32, device=dev),
                "tables": meta[off:off + 256 * nt],
                "code_len": meta[off + 256 * nt:off + 256 * nt + 256],
                "n_tables": nt, "total_bits": int(c["total_bits"]),
                "shape": tuple(m.shape)})
            off += 256 * nt + 256
        ws = _workspace(_lib.OP_DF11_ENCODE, mats, 0, ws, dev)
    cl = [np.ascontiguousarray(c["code_len"], dtype=np.uint8) for c in codes]
    cw = [np.ascontiguousarray(c["codeword"], dtype=np.uint32) for c in codes]
    tb = (ctypes.c_int64 * len(mats))(*[c["total_bits"] for c in codes])
    st = lib.df11_encode(arr, len(mats), _host_ptrs(cl), _host_ptrs(cw), tb,
                         _ptrs([o["enc"] for o in outs]), _ptrs([o["sm"] for o in outs]),
                         _ptrs([o["gaps"] for o in outs]), _ptrs([o["block_pos"] for o in outs]),
                         ws.data_ptr(), ws.numel(), _stream(stream, dev))
    _lib.check("df11_encode", st)
    return outs


def df11_compress(mats: Sequence[torch.Tensor], *, hist=None, stream=None):
    """Histogram (device; skipped when ``hist`` [n_mats, 256] is given, for
    example the exponent histograms of the entropy pass), codes (host; one
    synchronisation), encode (device)."""
    if hist is None:
        hist = df11_exponent_histogram(mats, stream=stream)
    if isinstance(hist, torch.Tensor):
        hist = hist.cpu().numpy()
    if len(hist) != len(mats):
        raise ValueError(f"hist: {len(hist)} histograms for {len(mats)} matrices")
    codes = [df11_build_code(h) for h in hist]
    return df11_encode(mats, codes, stream=stream)


def df11_decode(encoded, *, out=None, ws=None, stream=None):
    """Exact bf16 weights of a batch of encoded matrices (one launch)."""
    lib = _lib.load()
    if len(encoded) == 0:
        raise ValueError("at least one encoded matrix is required")
    if out is not None and [tuple(o.shape) for o in out] != [tuple(e["shape"]) for e in encoded]:
        raise ValueError("out: tensors do not have the encoded shapes")
    dev = _device([e[k] for e in encoded for k in ("enc", "sm", "gaps", "block_pos", "tables",
                                                    "code_len")], out, ws)
    with _on(stream, dev):
        if out is None:
            out = [torch.empty(e["shape"], dtype=torch.bfloat16, device=dev) for e in encoded]
        arr = _mats(out)
        ws = _workspace(_lib.OP_DF11_DECODE, out, 0, ws, dev)
    nt = (ctypes.c_int32 * len(out))(*[e["n_tables"] for e in encoded])
    tb = (ctypes.c_int64 * len(out))(*[e["total_bits"] for e in encoded])
    st = lib.df11_decode(arr, len(out), _ptrs([e["enc"] for e in encoded]),
                         _ptrs([e["sm"] for e in encoded]), _ptrs([e["gaps"] for e in encoded]),
                         _ptrs([e["block_pos"] for e in encoded]),
                         _ptrs([e["tables"] for e in encoded]), nt,
                         _ptrs([e["code_len"] for e in encoded]), tb,
                         ws.data_ptr(), ws.numel(), _stream(stream, dev))
    _lib.check("df11_decode", st)
    return out
