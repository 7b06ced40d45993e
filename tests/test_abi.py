"""The C-ABI library loads and exports what include/dsa.h declares; host-side
argument checks answer without touching a GPU (no compute calls here)."""

import ctypes
import os
import re

import pytest

from sparse_attention_index_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_attention_index_amd.build import build

        build()
    return _lib.load()


def _declared():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(_lib.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.dsa_version() >= 100
    assert lib.dsa_status_string(0) == b"ok"
    for code in (-1, -2, -3, -4):
        assert lib.dsa_status_string(code) not in (b"ok", b"unknown status")


def test_workspace_sizes(lib):
    assert lib.dsa_workspace_size(_lib.DSA_WS_TOPK, 0, 1000, 2048, 16) == 0
    t1 = lib.dsa_workspace_size(_lib.DSA_WS_TOPK, 64, 32768, 2048, 16)
    t2 = lib.dsa_workspace_size(_lib.DSA_WS_TOPK, 64, 1 << 20, 2048, 16)
    assert 0 < t1 <= t2
    assert lib.dsa_workspace_size(_lib.DSA_WS_TOPK, 128, 32768, 2048, 16) > t1
    d = lib.dsa_workspace_size(_lib.DSA_WS_DECODE, 64, 32768, 2048, 16)
    assert d >= 64 * 32768 * 4 + 64 * 2048 * 4  # scores + selection at least
    assert lib.dsa_workspace_size(_lib.DSA_WS_MLA_PREFILL, 4096, 0, 2048, 16) == 0
    assert lib.dsa_workspace_size(99, 4, 100, 64, 16) == 0


def _batch(**kw):
    b = dict(num_requests=1, rows_per_request=1, ctx_len=1, block_table=1, max_blocks=1, max_ctx=64)
    b.update(kw)
    return _lib.DsaBatchC(b["num_requests"], b["rows_per_request"], b["ctx_len"], b["block_table"],
                          b["max_blocks"], b["max_ctx"])


def _cache(**kw):
    c = dict(key_fp8=256, key_scale=256, lat_fp8=256, lat_scale=256, num_blocks=1, block_size=64)
    c.update(kw)
    return _lib.DsaCacheC(c["key_fp8"], c["key_scale"], c["lat_fp8"], c["lat_scale"], c["num_blocks"],
                          c["block_size"])


def test_argument_errors_are_reported_before_any_launch(lib):
    P = 256  # a non-null, aligned host-side stand-in; never dereferenced on these error paths
    b, c = _batch(), _cache()
    assert lib.dsa_index_score(None, ctypes.byref(c), P, 0, None, P, P, 64, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_index_score(ctypes.byref(b), ctypes.byref(_cache(block_size=128)), P, 0, None, P, P, 64,
                               None) == _lib.DSA_ERR_UNSUPPORTED
    assert lib.dsa_index_score(ctypes.byref(b), ctypes.byref(c), P, 0, P, P, P, 64, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_index_score(ctypes.byref(b), ctypes.byref(c), P, 1, None, P, P, 64, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_index_score(ctypes.byref(b), ctypes.byref(c), P, 7, None, P, P, 64, None) == _lib.DSA_ERR_UNSUPPORTED
    assert lib.dsa_index_score(ctypes.byref(b), ctypes.byref(c), P, 0, None, P, P, 63, None) == _lib.DSA_ERR_INVALID_ARG
    assert b"ld" in lib.dsa_last_error()
    bad = _batch(max_blocks=1, max_ctx=65)
    assert lib.dsa_index_score(ctypes.byref(bad), ctypes.byref(c), P, 0, None, P, P, 65, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_index_score(ctypes.byref(_batch(rows_per_request=0)), ctypes.byref(c), P, 0, None, P, P, 64,
                               None) == _lib.DSA_ERR_INVALID_ARG
    # top-k
    assert lib.dsa_topk(P, 64, P, 4, 0, P, P, 1 << 30, None) == _lib.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(P, 64, P, 4, 2049, P, P, 1 << 30, None) == _lib.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(P, 64, P, 0, 64, P, P, 0, None) == _lib.DSA_OK  # nothing to do
    assert lib.dsa_topk(P, 64, P, 4, 64, P, P, 16, None) == _lib.DSA_ERR_WORKSPACE
    assert lib.dsa_topk(None, 64, P, 4, 64, P, P, 1 << 30, None) == _lib.DSA_ERR_INVALID_ARG
    # attention
    for fn in (lib.dsa_sparse_mla_decode, lib.dsa_sparse_mla_prefill):
        assert fn(ctypes.byref(b), ctypes.byref(c), P, 12, P, 64, 0.1, P, None, P, 1 << 30, None) == \
            _lib.DSA_ERR_UNSUPPORTED
        assert fn(ctypes.byref(b), ctypes.byref(c), P, 16, P, 0, 0.1, P, None, P, 1 << 30, None) == \
            _lib.DSA_ERR_UNSUPPORTED
        assert fn(ctypes.byref(b), ctypes.byref(c), P, 16, None, 64, 0.1, P, None, P, 1 << 30, None) == \
            _lib.DSA_ERR_INVALID_ARG
        assert fn(ctypes.byref(b), ctypes.byref(c), P + 2, 16, P, 64, 0.1, P, None, P, 1 << 30, None) == \
            _lib.DSA_ERR_INVALID_ARG
    # index-key write
    kw = lib.dsa_index_key_write
    assert kw(None, P, P, P, 1e-6, P, P, 1, None) == _lib.DSA_ERR_INVALID_ARG
    assert kw(ctypes.byref(b), None, P, P, 1e-6, P, P, 1, None) == _lib.DSA_ERR_INVALID_ARG
    assert kw(ctypes.byref(b), P, P, P, 0.0, P, P, 1, None) == _lib.DSA_ERR_INVALID_ARG
    assert kw(ctypes.byref(b), P, P, P, float("nan"), P, P, 1, None) == _lib.DSA_ERR_INVALID_ARG
    assert kw(ctypes.byref(b), P, P, P, 1e-6, P, P, 0, None) == _lib.DSA_ERR_INVALID_ARG
    assert kw(ctypes.byref(b), P + 2, P, P, 1e-6, P, P, 1, None) == _lib.DSA_ERR_INVALID_ARG
    # fused decode
    BF, F8 = _lib.DSA_Q_BF16, _lib.DSA_Q_FP8
    assert lib.dsa_decode(ctypes.byref(b), ctypes.byref(c), P, BF, None, P, P, 16, 2048, 0.1, P, None, None, P, 16,
                          None) == _lib.DSA_ERR_WORKSPACE
    assert lib.dsa_decode(ctypes.byref(b), ctypes.byref(_cache(lat_fp8=0)), P, BF, None, P, P, 16, 2048, 0.1, P, None,
                          None, P, 1 << 30, None) == _lib.DSA_ERR_INVALID_ARG
    # the indexer query's format: FP8 codes need their row scales, bf16 takes none
    assert lib.dsa_decode(ctypes.byref(b), ctypes.byref(c), P, F8, None, P, P, 16, 2048, 0.1, P, None, None, P,
                          1 << 30, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_decode(ctypes.byref(b), ctypes.byref(c), P, BF, P, P, P, 16, 2048, 0.1, P, None, None, P,
                          1 << 30, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_decode(ctypes.byref(b), ctypes.byref(c), P, 7, None, P, P, 16, 2048, 0.1, P, None, None, P,
                          1 << 30, None) == _lib.DSA_ERR_UNSUPPORTED
    assert lib.dsa_filter_score(ctypes.byref(b), ctypes.byref(c), P, F8, None, P, 2048, P, 1 << 30, None) == \
        _lib.DSA_ERR_INVALID_ARG


def test_binding_refuses_host_tensors():
    """Tensor checks in the binding run before the library is called."""
    import torch

    import sparse_attention_index_amd as dsa

    ctx = torch.tensor([100], dtype=torch.int32)
    table = torch.zeros((1, 2), dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        dsa.Batch(1, ctx, table, 100)
