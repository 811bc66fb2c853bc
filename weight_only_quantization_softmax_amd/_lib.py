"""ctypes view of libwoq.so: the C ABI declared in include/woq.h.

Argument marshalling only.  The library must be built in-tree
(``python -m weight_only_quantization_softmax_amd.build``); there is no
fallback of any kind when it is missing.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwoq.so")

WOQ_OK = 0
STATUS = {
    0: "WOQ_OK", 1: "WOQ_ERR_NULL", 2: "WOQ_ERR_SHAPE", 3: "WOQ_ERR_DTYPE",
    4: "WOQ_ERR_BITS", 5: "WOQ_ERR_ITERS", 6: "WOQ_ERR_WORKSPACE",
    7: "WOQ_ERR_BLOCK", 8: "WOQ_ERR_HIP", 9: "WOQ_ERR_ALIGN", 10: "WOQ_ERR_COUNT",
    11: "WOQ_ERR_VALUE", 12: "WOQ_ERR_SCRATCH",
}
WOQ_F32, WOQ_BF16 = 0, 1
WOQ_SINQ_RMS = 1
WOQ_SINQ_SHARED = 2
OP_ENTROPY, OP_SINQ, OP_QUANT, OP_DEQUANT, OP_TERNARY = 1, 2, 3, 4, 5
OP_DF11_HIST, OP_DF11_ENCODE, OP_DF11_DECODE = 6, 7, 8

# every symbol include/woq.h declares
EXPORTS = ("woq_status_string", "woq_workspace_size", "ewq_block_entropy",
           "sinq_balance", "sinq_balance_ex", "quant_pack_groupwise", "dequant_unpack", "ternary_pack",
           "ewq_budget_levels", "df11_buffer_sizes", "df11_exponent_histogram",
           "df11_build_code", "df11_encode", "df11_decode", "quant_pack_codebook",
           "dequant_codebook", "woq_codebook_normal", "ewq_block_entropy_static",
           "ewq_block_entropy_ex")


WS_HEAD = 256   # WOQ_WS_HEAD: the workspace's status head (non-finite count at byte 0)


class WoqMat(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld", ctypes.c_int64)]


class WoqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


_lib = None

P = ctypes.c_void_p
PP = ctypes.POINTER(ctypes.c_void_p)
I32 = ctypes.c_int32


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m weight_only_quantization_softmax_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.woq_status_string.argtypes = [I32]
    lib.woq_status_string.restype = ctypes.c_char_p
    lib.woq_workspace_size.argtypes = [I32, ctypes.POINTER(WoqMat), I32, I32,
                                       ctypes.POINTER(ctypes.c_size_t)]
    lib.woq_workspace_size.restype = I32
    lib.ewq_block_entropy.argtypes = [ctypes.POINTER(WoqMat), I32, ctypes.POINTER(I32), I32,
                                      ctypes.c_double, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.ewq_block_entropy.restype = I32
    lib.ewq_block_entropy_ex.argtypes = [ctypes.POINTER(WoqMat), I32, ctypes.POINTER(I32), I32,
                                         ctypes.c_double, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.ewq_block_entropy_ex.restype = I32
    lib.ewq_block_entropy_static.argtypes = [ctypes.POINTER(WoqMat), I32, ctypes.POINTER(I32), I32,
                                             ctypes.c_double, P, P, P, P, P, P]
    lib.ewq_block_entropy_static.restype = I32
    lib.sinq_balance.argtypes = [ctypes.POINTER(WoqMat), I32, I32, PP, PP, P, ctypes.c_size_t, P]
    lib.sinq_balance.restype = I32
    lib.sinq_balance_ex.argtypes = [ctypes.POINTER(WoqMat), I32, I32, I32, PP, PP, P,
                                    ctypes.c_size_t, P]
    lib.sinq_balance_ex.restype = I32
    lib.quant_pack_groupwise.argtypes = [ctypes.POINTER(WoqMat), I32, PP, PP, I32, I32,
                                         PP, PP, PP, P, ctypes.c_size_t, P]
    lib.quant_pack_groupwise.restype = I32
    lib.dequant_unpack.argtypes = [ctypes.POINTER(WoqMat), I32, PP, PP, PP, PP, PP, I32, I32,
                                   P, ctypes.c_size_t, P]
    lib.dequant_unpack.restype = I32
    lib.ternary_pack.argtypes = [ctypes.POINTER(WoqMat), I32, PP, PP, P, ctypes.c_size_t, P]
    lib.ternary_pack.restype = I32
    lib.ewq_budget_levels.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
                                      I32, I32, ctypes.POINTER(I32), ctypes.c_int64,
                                      ctypes.POINTER(I32), ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(I32)]
    lib.ewq_budget_levels.restype = I32
    I64P = ctypes.POINTER(ctypes.c_int64)
    lib.df11_buffer_sizes.argtypes = [ctypes.c_int64, ctypes.c_int64, I64P, I64P, I64P, I64P]
    lib.df11_buffer_sizes.restype = I32
    lib.df11_exponent_histogram.argtypes = [ctypes.POINTER(WoqMat), I32, P, P, ctypes.c_size_t, P]
    lib.df11_exponent_histogram.restype = I32
    lib.df11_build_code.argtypes = [I64P, P, P, P, ctypes.POINTER(I32), I64P]
    lib.df11_build_code.restype = I32
    lib.df11_encode.argtypes = [ctypes.POINTER(WoqMat), I32, PP, PP, I64P, PP, PP, PP, PP,
                                P, ctypes.c_size_t, P]
    lib.df11_encode.restype = I32
    lib.df11_decode.argtypes = [ctypes.POINTER(WoqMat), I32, PP, PP, PP, PP, PP,
                                ctypes.POINTER(I32), PP, I64P, P, ctypes.c_size_t, P]
    lib.df11_decode.restype = I32
    FP = ctypes.POINTER(ctypes.c_float)
    lib.quant_pack_codebook.argtypes = [ctypes.POINTER(WoqMat), I32, PP, PP, I32, I32, FP,
                                        PP, PP, P, ctypes.c_size_t, P]
    lib.quant_pack_codebook.restype = I32
    lib.dequant_codebook.argtypes = [ctypes.POINTER(WoqMat), I32, PP, PP, PP, PP, I32, I32, FP,
                                     P, ctypes.c_size_t, P]
    lib.dequant_codebook.restype = I32
    lib.woq_codebook_normal.argtypes = [I32, FP]
    lib.woq_codebook_normal.restype = I32
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != WOQ_OK:
        raise WoqError(fn, status)


# numpy view of the woq_mat layout (filled column-wise, then shared with a
# ctypes array without a copy)
_MAT_NP = np.dtype({"names": ["data", "dtype", "reserved", "rows", "cols", "ld"],
                    "formats": ["<u8", "<i4", "<i4", "<i8", "<i8", "<i8"],
                    "offsets": [0, 8, 12, 16, 24, 32], "itemsize": ctypes.sizeof(WoqMat)})


def mat_array(descs):
    """descs: iterable of (data_ptr, dtype, rows, cols[, ld]) -> ctypes WoqMat
    array (ld 0 = contiguous)."""
    descs = list(descs)
    a = np.zeros(len(descs), dtype=_MAT_NP)
    if descs:
        a["data"] = [d[0] or 0 for d in descs]
        a["dtype"] = [d[1] for d in descs]
        a["rows"] = [d[2] for d in descs]
        a["cols"] = [d[3] for d in descs]
        a["ld"] = [d[4] if len(d) > 4 else 0 for d in descs]
    return (WoqMat * len(descs)).from_buffer(a)


def ptr_array(ptrs):
    """Host array of device pointers (None entries become NULL); None -> NULL array."""
    if ptrs is None:
        return None
    ptrs = list(ptrs)
    arr = (ctypes.c_void_p * len(ptrs))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return ctypes.cast(arr, PP)
