"""Python binding of libdsa, the gfx950 DSA hot path (Score -> Select -> Attend).

Every function here only marshals torch tensors (device memory) and the
current HIP stream into the C ABI of include/dsa.h; all arithmetic runs in the
HIP kernels. The functions carry the C names. There is no fallback: if
libdsa.so was not built, `load()` raises.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import (  # noqa: F401
    DSA_ERR_HIP,
    DSA_ERR_INVALID_ARG,
    DSA_ERR_UNSUPPORTED,
    DSA_ERR_WORKSPACE,
    DSA_OK,
    DSA_Q_BF16,
    DSA_Q_FP8,
    DSA_WS_DECODE,
    DSA_WS_MLA_DECODE,
    DSA_WS_MLA_PREFILL,
    DSA_WS_TOPK,
    EXPORTS,
    LIB_PATH,
)


class DsaError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what} failed: {detail or 'status ' + str(status)} ({status})")
        self.status = status


def load():
    return _lib.load()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str):
    if status != DSA_OK:
        lib = load()
        detail = lib.dsa_last_error().decode() or lib.dsa_status_string(status).decode()
        raise DsaError(status, what, detail)


class Cache:
    """Paged cache planes (device tensors): key_fp8 u8 [nb,64,128], key_scale f32 [nb,64],
    lat_fp8 u8 [nb,64,576], lat_scale f32 [nb,64]."""

    def __init__(self, key_fp8, key_scale, lat_fp8, lat_scale):
        self.key_fp8, self.key_scale, self.lat_fp8, self.lat_scale = key_fp8, key_scale, lat_fp8, lat_scale
        nb = key_fp8.shape[0] if key_fp8 is not None else lat_fp8.shape[0]
        self.c = _lib.DsaCacheC(
            _ptr(key_fp8), _ptr(key_scale), _ptr(lat_fp8), _ptr(lat_scale), int(nb), 64
        )

    @classmethod
    def of(cls, case) -> "Cache":
        return cls(case.key_fp8, case.key_scale, case.lat_fp8, case.lat_scale)


class Batch:
    """ctx_len int32 [B] and block_table int32 [B, max_blocks] on the device;
    max_ctx is a host-side bound of ctx_len."""

    def __init__(self, rows_per_request: int, ctx_len, block_table, max_ctx: int):
        self.ctx_len, self.block_table = ctx_len, block_table
        self.R = int(rows_per_request)
        self.B = int(ctx_len.shape[0])
        self.max_ctx = int(max_ctx)
        self.c = _lib.DsaBatchC(
            self.B, self.R, _ptr(ctx_len), _ptr(block_table), int(block_table.shape[1]), self.max_ctx
        )

    @property
    def rows(self) -> int:
        return self.B * self.R

    @classmethod
    def of(cls, case) -> "Batch":
        return cls(case.R, case.ctx_len, case.block_table, case.max_ctx)


def dsa_workspace_size(kind: int, rows: int, max_ctx: int, k: int, num_heads: int = 16) -> int:
    return int(load().dsa_workspace_size(kind, rows, max_ctx, k, num_heads))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def dsa_index_score(batch: Batch, cache: Cache, q, w, scores, q_scale=None, stream=None):
    """scores[row, s] for every visible token s (fp32 [rows, ld])."""
    q_dtype = DSA_Q_FP8 if q_scale is not None else DSA_Q_BF16
    st = load().dsa_index_score(
        ctypes.byref(batch.c), ctypes.byref(cache.c), _ptr(q), q_dtype, _ptr(q_scale), _ptr(w),
        _ptr(scores), int(scores.stride(0)), _stream(stream),
    )
    _check(st, "dsa_index_score")


def dsa_topk(scores, row_len, k: int, idx, ws, stream=None):
    """idx[row, :] = positions of the k largest scores[row, :row_len[row]] (set; -1 padded)."""
    rows = int(scores.shape[0])
    st = load().dsa_topk(
        _ptr(scores), int(scores.stride(0)), _ptr(row_len), rows, int(k), _ptr(idx),
        _ptr(ws), int(ws.numel()) if ws is not None else 0, _stream(stream),
    )
    _check(st, "dsa_topk")


def _mla(fn, name, batch, cache, q, idx, softmax_scale, out, lse, ws, stream):
    st = fn(
        ctypes.byref(batch.c), ctypes.byref(cache.c), _ptr(q), int(q.shape[1]), _ptr(idx), int(idx.shape[1]),
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws), int(ws.numel()) if ws is not None else 0,
        _stream(stream),
    )
    _check(st, name)


def dsa_sparse_mla_decode(batch, cache, q, idx, softmax_scale, out, lse=None, ws=None, stream=None):
    _mla(load().dsa_sparse_mla_decode, "dsa_sparse_mla_decode", batch, cache, q, idx, softmax_scale, out, lse,
         ws, stream)


def dsa_sparse_mla_prefill(batch, cache, q, idx, softmax_scale, out, lse=None, ws=None, stream=None):
    _mla(load().dsa_sparse_mla_prefill, "dsa_sparse_mla_prefill", batch, cache, q, idx, softmax_scale, out, lse,
         ws, stream)


def dsa_decode(batch, cache, q_idx, w, q_mla, k, softmax_scale, out, lse=None, idx_out=None, ws=None,
               stream=None):
    st = load().dsa_decode(
        ctypes.byref(batch.c), ctypes.byref(cache.c), _ptr(q_idx), _ptr(w), _ptr(q_mla), int(q_mla.shape[1]),
        int(k), float(softmax_scale), _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws),
        int(ws.numel()) if ws is not None else 0, _stream(stream),
    )
    _check(st, "dsa_decode")
