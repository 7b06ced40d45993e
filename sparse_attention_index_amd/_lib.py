"""ctypes view of libdsa.so (declarations in include/dsa.h)."""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK = 0
DSA_ERR_INVALID_ARG = -1
DSA_ERR_UNSUPPORTED = -2
DSA_ERR_WORKSPACE = -3
DSA_ERR_HIP = -4
DSA_Q_BF16 = 0
DSA_Q_FP8 = 1
DSA_WS_TOPK = 1
DSA_WS_MLA_DECODE = 2
DSA_WS_MLA_PREFILL = 3
DSA_WS_DECODE = 4
DSA_WS_DCP_TOPK = 5
DSA_WS_DCP_MLA = 6

EXPORTS = (
    "dsa_index_key_write",
    "dsa_index_score",
    "dsa_topk",
    "dsa_sparse_mla_decode",
    "dsa_sparse_mla_prefill",
    "dsa_sparse_mla_decode_noalloc",
    "dsa_decode",
    "dsa_decode_thresholded",
    "dsa_filter_threshold",
    "dsa_filter_score",
    "dsa_filter_select",
    "dsa_workspace_size",
    "dsa_dcp_topk",
    "dsa_dcp_mla_decode",
    "dsa_dcp_workspace_size",
    "dsa_status_string",
    "dsa_last_error",
    "dsa_version",
)


class DsaCacheC(ctypes.Structure):
    _fields_ = [
        ("key_fp8", ctypes.c_void_p),
        ("key_scale", ctypes.c_void_p),
        ("lat_fp8", ctypes.c_void_p),
        ("lat_scale", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("key_format", ctypes.c_int32),
        ("key_fp4", ctypes.c_void_p),
        ("key_e8m0", ctypes.c_void_p),
    ]


class DsaBatchC(ctypes.Structure):
    _fields_ = [
        ("num_requests", ctypes.c_int32),
        ("rows_per_request", ctypes.c_int32),
        ("ctx_len", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("max_blocks", ctypes.c_int32),
        ("max_ctx", ctypes.c_int32),
    ]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsa.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m sparse_attention_index_amd.build` "
            "(there is no fallback implementation)"
        )
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I32 = ctypes.c_int32
    I64 = ctypes.c_int64
    SZ = ctypes.c_size_t
    F = ctypes.c_float
    BP = ctypes.POINTER(DsaBatchC)
    CP = ctypes.POINTER(DsaCacheC)
    sig = {
        "dsa_index_key_write": (I32, [BP, P, P, P, F, P, P, I32, P]),
        "dsa_index_score": (I32, [BP, CP, P, I32, P, P, P, I64, P]),
        "dsa_topk": (I32, [P, I64, P, I32, I32, P, P, SZ, P]),
        "dsa_sparse_mla_decode": (I32, [BP, CP, P, I32, P, I32, F, P, P, P, SZ, P]),
        "dsa_sparse_mla_prefill": (I32, [BP, CP, P, I32, P, I32, F, P, P, P, SZ, P]),
        "dsa_sparse_mla_decode_noalloc": (I32, [BP, CP, P, I32, P, I32, F, P, P, P]),
        "dsa_decode": (I32, [BP, CP, P, I32, P, P, P, I32, I32, F, P, P, P, P, SZ, P]),
        "dsa_decode_thresholded": (I32, [BP, CP, P, I32, P, P, P, I32, I32, F, P, P, P, P, P, SZ, P]),
        "dsa_filter_threshold": (I32, [BP, CP, P, I32, P, P, I32, P, P, SZ, P]),
        "dsa_filter_score": (I32, [BP, CP, P, I32, P, P, I32, P, SZ, P]),
        "dsa_filter_select": (I32, [BP, CP, P, I32, P, P, I32, P, P, SZ, P]),
        "dsa_workspace_size": (SZ, [I32, I32, I64, I32, I32]),
        "dsa_dcp_topk": (I32, [P, I64, P, I32, I32, I32, I32, P, P, P, SZ, P]),
        "dsa_dcp_mla_decode": (I32, [BP, CP, P, I32, P, I32, I32, F, P, P, P, SZ, P]),
        "dsa_dcp_workspace_size": (SZ, [I32, I32, I64, I32, I32, I32]),
        "dsa_status_string": (ctypes.c_char_p, [I32]),
        "dsa_last_error": (ctypes.c_char_p, []),
        "dsa_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
