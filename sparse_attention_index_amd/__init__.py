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
    DSA_WS_DCP_MLA,
    DSA_WS_DCP_TOPK,
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


def _need(t, name: str, dtypes, numel: int = 0, contiguous: bool = True):
    """Tensor checks the C ABI cannot make (it sees raw pointers): device, dtype, size, layout."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {tuple(dtypes)}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF16 = (torch.bfloat16,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)
_CODES = (torch.uint8, torch.float8_e4m3fn)


def _check_scores(scores, rows: int, cols: int):
    _need(scores, "scores", _F32, contiguous=False)
    if scores.dim() != 2 or scores.stride(1) != 1 or scores.shape[0] < rows or scores.shape[1] < cols:
        raise ValueError(f"scores must be fp32 [>= {rows}, >= {cols}] with unit column stride")


def _check(status: int, what: str):
    if status != DSA_OK:
        lib = load()
        detail = lib.dsa_last_error().decode() or lib.dsa_status_string(status).decode()
        raise DsaError(status, what, detail)


DSA_KEY_FP8 = 0
DSA_KEY_MXFP4 = 1


class Cache:
    """Paged cache planes (device tensors): key_fp8 u8 [nb,64,128], key_scale f32 [nb,64],
    lat_fp8 u8 [nb,64,576], lat_scale f32 [nb,64]; or, for MXFP4 index keys,
    key_fp4 u8 [nb,64,64] (E2M1 pairs, even dim in the low nibble) and
    key_e8m0 u8 [nb,64,4] in place of key_fp8 / key_scale."""

    def __init__(self, key_fp8, key_scale, lat_fp8, lat_scale, key_fp4=None, key_e8m0=None):
        if key_fp8 is not None and key_fp4 is not None:
            raise ValueError("give FP8 or MXFP4 key planes, not both")
        nb = None
        if key_fp8 is not None:
            _need(key_fp8, "key_fp8", _CODES)
            nb = key_fp8.shape[0]
            if tuple(key_fp8.shape[1:]) != (64, 128):
                raise ValueError("key_fp8 must be [num_blocks, 64, 128]")
            _need(key_scale, "key_scale", _F32, nb * 64)
        if key_fp4 is not None:
            _need(key_fp4, "key_fp4", _CODES)
            nb = key_fp4.shape[0]
            if tuple(key_fp4.shape[1:]) != (64, 64):
                raise ValueError("key_fp4 must be [num_blocks, 64, 64]")
            _need(key_e8m0, "key_e8m0", _CODES, nb * 64 * 4)
        if lat_fp8 is not None:
            _need(lat_fp8, "lat_fp8", _CODES)
            if tuple(lat_fp8.shape[1:]) != (64, 576):
                raise ValueError("lat_fp8 must be [num_blocks, 64, 576]")
            _need(lat_scale, "lat_scale", _F32, lat_fp8.shape[0] * 64)
            if nb is not None and lat_fp8.shape[0] != nb:
                raise ValueError("key and latent planes must have the same number of blocks")
        self.key_fp8, self.key_scale, self.lat_fp8, self.lat_scale = key_fp8, key_scale, lat_fp8, lat_scale
        self.key_fp4, self.key_e8m0 = key_fp4, key_e8m0
        if nb is None:
            nb = lat_fp8.shape[0]
        fmt = DSA_KEY_MXFP4 if key_fp4 is not None else DSA_KEY_FP8
        self.c = _lib.DsaCacheC(
            _ptr(key_fp8), _ptr(key_scale), _ptr(lat_fp8), _ptr(lat_scale), int(nb), 64, fmt, _ptr(key_fp4),
            _ptr(key_e8m0)
        )

    @classmethod
    def of(cls, case) -> "Cache":
        return cls(case.key_fp8, case.key_scale, case.lat_fp8, case.lat_scale,
                   getattr(case, "key_fp4", None), getattr(case, "key_e8m0", None))


class Batch:
    """ctx_len int32 [B] and block_table int32 [B, max_blocks] on the device;
    max_ctx is a host-side bound of ctx_len."""

    def __init__(self, rows_per_request: int, ctx_len, block_table, max_ctx: int):
        _need(ctx_len, "ctx_len", _I32)
        _need(block_table, "block_table", _I32)
        if block_table.dim() != 2 or block_table.shape[0] != ctx_len.shape[0]:
            raise ValueError("block_table must be [num_requests, max_blocks]")
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


def dsa_dcp_workspace_size(kind: int, rows: int, ld: int, k: int, W: int, C: int = 0) -> int:
    return int(load().dsa_dcp_workspace_size(kind, rows, ld, k, W, C))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def dsa_index_key_write(batch: Batch, k, ln_weight, ln_bias, key_fp8, key_scale, eps: float = 1e-6, stream=None):
    """Write the batch's new rows' index keys into the cache planes: LayerNorm
    of k (bf16 [rows, 128]) with ln_weight / ln_bias (fp32 [128]), E4M3
    quantisation with one absmax scale per row, paged by the batch's tables.
    key_fp8 (uint8 [nb, 64, 128]) and key_scale (fp32 [nb, 64]) are written in place."""
    rows = batch.rows
    _need(k, "k", _BF16, rows * 128)
    _need(ln_weight, "ln_weight", _F32, 128)
    _need(ln_bias, "ln_bias", _F32, 128)
    _need(key_fp8, "key_fp8", _CODES)
    if key_fp8.dim() != 3 or tuple(key_fp8.shape[1:]) != (64, 128):
        raise ValueError("key_fp8 must be [num_blocks, 64, 128]")
    nb = int(key_fp8.shape[0])
    _need(key_scale, "key_scale", _F32, nb * 64)
    st = load().dsa_index_key_write(
        ctypes.byref(batch.c), _ptr(k), _ptr(ln_weight), _ptr(ln_bias), float(eps), _ptr(key_fp8), _ptr(key_scale),
        nb, _stream(stream),
    )
    _check(st, "dsa_index_key_write")


def _index_query(q, q_scale, w, rows, name="q"):
    """The indexer query's format: bf16, or E4M3 codes with fp32 row scales."""
    if q_scale is None:
        _need(q, name, _BF16, rows * 32 * 128)
    else:
        _need(q, name, _CODES, rows * 32 * 128)
        _need(q_scale, "q_scale", _F32, rows)
    _need(w, "w", _BF16, rows * 32)
    return DSA_Q_FP8 if q_scale is not None else DSA_Q_BF16


def dsa_index_score(batch: Batch, cache: Cache, q, w, scores, q_scale=None, stream=None):
    """scores[row, s] for every visible token s (fp32 [rows, ld])."""
    rows = batch.rows
    q_dtype = _index_query(q, q_scale, w, rows)
    _check_scores(scores, rows, batch.max_ctx)
    st = load().dsa_index_score(
        ctypes.byref(batch.c), ctypes.byref(cache.c), _ptr(q), q_dtype, _ptr(q_scale), _ptr(w),
        _ptr(scores), int(scores.stride(0)), _stream(stream),
    )
    _check(st, "dsa_index_score")


def dsa_topk(scores, row_len, k: int, idx, ws, stream=None):
    """idx[row, :] = positions of the k largest scores[row, :row_len[row]] (set; -1 padded)."""
    rows = int(scores.shape[0])
    _check_scores(scores, rows, 1)
    _need(row_len, "row_len", _I32, rows)
    _need(idx, "idx", _I32, rows * int(k))
    if ws is not None:
        _need(ws, "ws", (torch.uint8,))
    st = load().dsa_topk(
        _ptr(scores), int(scores.stride(0)), _ptr(row_len), rows, int(k), _ptr(idx),
        _ptr(ws), int(ws.numel()) if ws is not None else 0, _stream(stream),
    )
    _check(st, "dsa_topk")


def dsa_dcp_topk(scores, row_len, k: int, W: int, C: int, idx, resend, ws, stream=None):
    """The exact top-k merged across W virtual shards (token p on shard p mod W);
    idx as dsa_topk, resend uint8 [rows, W]."""
    rows = int(scores.shape[0])
    _check_scores(scores, rows, 1)
    _need(row_len, "row_len", _I32, rows)
    _need(idx, "idx", _I32, rows * int(k))
    _need(resend, "resend", (torch.uint8,), rows * int(W))
    if ws is not None:
        _need(ws, "ws", (torch.uint8,))
    st = load().dsa_dcp_topk(
        _ptr(scores), int(scores.stride(0)), _ptr(row_len), rows, int(k), int(W), int(C), _ptr(idx), _ptr(resend),
        _ptr(ws), int(ws.numel()) if ws is not None else 0, _stream(stream),
    )
    _check(st, "dsa_dcp_topk")


def dsa_dcp_mla_decode(batch, cache, q, idx, W: int, softmax_scale, out, lse=None, ws=None, stream=None):
    """Each of W virtual shards attends over the entries of idx it owns; partials combined by LSE."""
    fn = load().dsa_dcp_mla_decode

    def call(b, c, qp, nh, ip, k, sm, op, lp, wp, wn, s):
        return fn(b, c, qp, nh, ip, k, int(W), sm, op, lp, wp, wn, s)

    _mla(call, "dsa_dcp_mla_decode", batch, cache, q, idx, softmax_scale, out, lse, ws, stream)


def _mla(fn, name, batch, cache, q, idx, softmax_scale, out, lse, ws, stream):
    rows = batch.rows
    _need(q, "q", _BF16)
    if q.dim() != 3 or q.shape[0] != rows or q.shape[2] != 576:
        raise ValueError(f"q must be bf16 [{rows}, heads, 576]")
    _need(idx, "idx", _I32)
    if idx.dim() != 2 or idx.shape[0] != rows:
        raise ValueError(f"idx must be int32 [{rows}, k]")
    _need(out, "out", _BF16, rows * int(q.shape[1]) * 512)
    if lse is not None:
        _need(lse, "lse", _F32, rows * int(q.shape[1]))
    if ws is not None:
        _need(ws, "ws", (torch.uint8,))
    st = fn(
        ctypes.byref(batch.c), ctypes.byref(cache.c), _ptr(q), int(q.shape[1]), _ptr(idx), int(idx.shape[1]),
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws), int(ws.numel()) if ws is not None else 0,
        _stream(stream),
    )
    _check(st, name)


def dsa_sparse_mla_decode(batch, cache, q, idx, softmax_scale, out, lse=None, ws=None, stream=None):
    _mla(load().dsa_sparse_mla_decode, "dsa_sparse_mla_decode", batch, cache, q, idx, softmax_scale, out, lse,
         ws, stream)


def dsa_sparse_mla_decode_noalloc(batch, cache, q, idx, softmax_scale, out, lse=None, stream=None):
    """dsa_sparse_mla_decode with the library's own static scratch (no workspace, no allocation)."""
    fn = load().dsa_sparse_mla_decode_noalloc

    def call(b, c, qp, nh, ip, k, sm, op, lp, wp, wn, s):
        return fn(b, c, qp, nh, ip, k, sm, op, lp, s)

    _mla(call, "dsa_sparse_mla_decode_noalloc", batch, cache, q, idx, softmax_scale, out, lse, None, stream)


def dsa_sparse_mla_prefill(batch, cache, q, idx, softmax_scale, out, lse=None, ws=None, stream=None):
    _mla(load().dsa_sparse_mla_prefill, "dsa_sparse_mla_prefill", batch, cache, q, idx, softmax_scale, out, lse,
         ws, stream)


def dsa_decode(batch, cache, q_idx, w, q_mla, k, softmax_scale, out, lse=None, idx_out=None, ws=None,
               stream=None, threshold=None, q_scale=None):
    """The whole decode step (score -> select -> attend). With `threshold`
    (fp32 [rows] on the device) the rows' candidate thresholds are the
    caller's (dsa_decode_thresholded) instead of sampled; results are the same.
    With `q_scale` (fp32 [rows]) q_idx holds E4M3 codes, else bf16 values."""
    rows = batch.rows
    q_dtype = _index_query(q_idx, q_scale, w, rows, "q_idx")
    _need(q_mla, "q_mla", _BF16)
    if q_mla.dim() != 3 or q_mla.shape[0] != rows or q_mla.shape[2] != 576:
        raise ValueError(f"q_mla must be bf16 [{rows}, heads, 576]")
    _need(out, "out", _BF16, rows * int(q_mla.shape[1]) * 512)
    if lse is not None:
        _need(lse, "lse", _F32, rows * int(q_mla.shape[1]))
    if idx_out is not None:
        _need(idx_out, "idx_out", _I32, rows * int(k))
    if ws is not None:
        _need(ws, "ws", (torch.uint8,))
    lib = load()
    head = (ctypes.byref(batch.c), ctypes.byref(cache.c), _ptr(q_idx), q_dtype, _ptr(q_scale), _ptr(w), _ptr(q_mla),
            int(q_mla.shape[1]), int(k), float(softmax_scale))
    tail = (_ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws), int(ws.numel()) if ws is not None else 0, _stream(stream))
    if threshold is None:
        _check(lib.dsa_decode(*head, *tail), "dsa_decode")
    else:
        _need(threshold, "threshold", _F32, rows)
        _check(lib.dsa_decode_thresholded(*head, _ptr(threshold), *tail), "dsa_decode_thresholded")


def _filter_head(batch, cache, q_idx, w, k, ws, q_scale):
    q_dtype = _index_query(q_idx, q_scale, w, batch.rows, "q_idx")
    _need(ws, "ws", (torch.uint8,))
    return (ctypes.byref(batch.c), ctypes.byref(cache.c), _ptr(q_idx), q_dtype, _ptr(q_scale), _ptr(w), int(k))


def dsa_filter_threshold(batch, cache, q_idx, w, k, ws, threshold=None, stream=None, q_scale=None):
    """Filtered path, stage 1: each row's candidate threshold (sampled, or
    `threshold`, fp32 [rows] on the device) into `ws` (dsa_decode's workspace)."""
    head = _filter_head(batch, cache, q_idx, w, k, ws, q_scale)
    if threshold is not None:
        _need(threshold, "threshold", _F32, batch.rows)
    _check(load().dsa_filter_threshold(*head, _ptr(threshold), _ptr(ws), int(ws.numel()), _stream(stream)),
           "dsa_filter_threshold")


def dsa_filter_score(batch, cache, q_idx, w, k, ws, stream=None, q_scale=None):
    """Filtered path, stage 2: the scores at or above each row's threshold, kept in `ws`."""
    head = _filter_head(batch, cache, q_idx, w, k, ws, q_scale)
    _check(load().dsa_filter_score(*head, _ptr(ws), int(ws.numel()), _stream(stream)), "dsa_filter_score")


def dsa_filter_select(batch, cache, q_idx, w, k, idx, ws, stream=None, q_scale=None):
    """Filtered path, stage 3: the exact top-k of every row into idx (int32 [rows, k])."""
    head = _filter_head(batch, cache, q_idx, w, k, ws, q_scale)
    _need(idx, "idx", _I32, batch.rows * int(k))
    _check(load().dsa_filter_select(*head, _ptr(idx), _ptr(ws), int(ws.numel()), _stream(stream)),
           "dsa_filter_select")
