"""Pins of the index-key write oracle (LayerNorm, E4M3 quantisation with one
absmax scale, paged write) against facts that do not come from the oracle:
torch's layer_norm and float8_e4m3fn cast as independent library routines,
closed forms, and the workloads' own quantiser; plus the mutants they catch.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.key_write as okw
from workloads.gen import quantize_e4m3_rows

RNG = np.random.default_rng(20260101)


def _rows(n=64, d=128, scale=1.0):
    return RNG.standard_normal((n, d)) * scale


# ---------------------------------------------------------------- LayerNorm


def test_layer_norm_matches_torch():
    x = _rows(32) * 3.0 + 0.5
    w = RNG.standard_normal(128)
    b = RNG.standard_normal(128)
    for eps in (1e-6, 1e-2):
        ref = torch.nn.functional.layer_norm(torch.tensor(x), (128,), torch.tensor(w), torch.tensor(b), eps).numpy()
        assert np.allclose(oracle.layer_norm(x, w, b, eps), ref, rtol=1e-12, atol=1e-12)


def test_layer_norm_closed_forms():
    w = np.linspace(0.5, 2.0, 128)
    b = np.linspace(-1.0, 1.0, 128)
    # a constant row has zero deviation: the output is the bias
    assert np.array_equal(oracle.layer_norm(np.full((1, 128), 7.25), w, b, 1e-6)[0], b)
    # +a, -a alternating: mean 0, biased variance a^2
    a, eps = 3.0, 1e-3
    x = np.where(np.arange(128) % 2 == 0, a, -a)[None, :]
    y = oracle.layer_norm(x, np.ones(128), np.zeros(128), eps)[0]
    assert np.allclose(y, x[0] / np.sqrt(a * a + eps), rtol=1e-14)
    # one spike in zeros: mean s/128, variance s^2 (127/128^2)
    s = 128.0
    x = np.zeros((1, 128))
    x[0, 5] = s
    y = oracle.layer_norm(x, np.ones(128), np.zeros(128), 0.0)[0]
    sd = s * np.sqrt(127.0) / 128.0
    assert np.isclose(y[5], (s - s / 128) / sd) and np.isclose(y[0], -(s / 128) / sd)


# ---------------------------------------------------------------- E4M3 encode


def _torch_e4m3(v32):
    return torch.tensor(v32, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_on_values_and_midpoints():
    tab = oracle.e4m3_table()
    finite = np.sort(np.unique(np.abs(tab[~np.isnan(tab)])))
    mids = (finite[:-1] + finite[1:]) / 2  # exact in float32: one more significant bit
    for vals in (finite, mids, -finite, -mids):
        v32 = vals.astype(np.float32)
        assert np.array_equal(oracle.e4m3_encode(v32), _torch_e4m3(v32))
    v = (RNG.standard_normal(200000) * RNG.choice([1e-3, 1.0, 60.0], 200000)).clip(-448, 448).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_encode_saturates_and_keeps_sign():
    codes = oracle.e4m3_encode(np.array([1e6, -1e6, 448.0, 464.0, -0.0, -1e-12, 0.0]))
    assert codes.tolist() == [0x7E, 0xFE, 0x7E, 0x7E, 0x80, 0x80, 0x00]


# ---------------------------------------------------------------- quantise rows


def test_quantize_rows_matches_the_workloads_quantiser():
    for scale in (1e-3, 1.0, 50.0):
        y = _rows(96, scale=scale).astype(np.float32)
        y[3] = 0.0  # all-zero row: scale 1
        codes, scales = oracle.quantize_rows(y)
        ref_codes, ref_scales = quantize_e4m3_rows(torch.tensor(y))
        assert np.array_equal(codes, ref_codes.numpy())
        assert np.array_equal(scales, ref_scales.numpy())
        assert scales[3] == 1.0 and not codes[3].any()


def test_quantized_row_reaches_the_end_of_the_range_and_stays_close():
    y = _rows(40, scale=5.0)
    codes, scales = oracle.quantize_rows(y)
    tab = oracle.e4m3_table()
    back = tab[codes] * scales[:, None]
    for r in range(40):
        assert np.abs(tab[codes[r]]).max() == 448.0  # the absmax element maps to the largest code
    # within half an E4M3 step: 2^-4 relative for normals, 2^-10 absolute (x scale) below 2^-6
    err = np.abs(back - y.astype(np.float32))
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10 * scales[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)


# ---------------------------------------------------------------- slots and scatter


def test_write_slots_hand_example():
    ctx = np.array([70, 3, 1])
    table = np.array([[4, 2, -1], [1, -1, -1], [-1, 0, 0]])
    # R = 2: request 0 rows at 68, 69 (page 1 -> block 2); request 1 at 1, 2
    # (page 0 -> block 1); request 2 at -1 (skipped) and 0 (page 0 -> -1, skipped)
    slots = oracle.write_slots(ctx, table, 2, num_blocks=5)
    assert slots.tolist() == [2 * 64 + 4, 2 * 64 + 5, 64 + 1, 64 + 2, -1, -1]
    # a block id past the pool is skipped too
    assert oracle.write_slots(np.array([1]), np.array([[9]]), 1, num_blocks=5).tolist() == [-1]


def test_scatter_rows_writes_only_the_slots():
    cp = np.zeros((3, 64, 128), np.uint8)
    sp = np.zeros((3, 64), np.float32)
    codes = np.full((2, 128), 0x38, np.uint8)
    ncp, nsp = oracle.scatter_rows(cp, sp, codes, np.array([2.0, 3.0], np.float32), np.array([65, -1]))
    assert ncp[1, 1].tolist() == [0x38] * 128 and nsp[1, 1] == 2.0
    ncp[1, 1] = 0
    nsp[1, 1] = 0
    assert not ncp.any() and not nsp.any() and not cp.any()


def test_index_key_write_hand_example():
    # k = 0..127: LayerNorm with unit weight, zero bias is (k - 63.5) / sd; the
    # largest magnitudes (k = 0 and 127) map to the end codes -448 / +448
    k = np.arange(128, dtype=np.float64)[None, :]
    codes, scales = oracle.index_key_write(k, np.ones(128), np.zeros(128), 1e-6)
    sd = np.sqrt(((k - 63.5) ** 2).mean() + 1e-6)
    assert np.isclose(scales[0], (63.5 / sd) / 448.0, rtol=1e-6)
    assert codes[0, 127] == 0x7E and codes[0, 0] == 0xFE
    # antisymmetric around the mean: code(k) and code(127 - k) differ in the sign bit only
    assert np.array_equal(codes[0, :64] ^ 0x80, codes[0, 64:][::-1])


# ---------------------------------------------------------------- mutants


def _ln_unbiased(x, w, b, eps):
    x = np.asarray(x, np.float64)
    m = x.mean(axis=-1, keepdims=True)
    v = ((x - m) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)
    return (x - m) / np.sqrt(v + eps) * w + b


def _ln_eps_outside(x, w, b, eps):
    x = np.asarray(x, np.float64)
    m = x.mean(axis=-1, keepdims=True)
    v = ((x - m) ** 2).mean(axis=-1, keepdims=True)
    return (x - m) / (np.sqrt(v) + eps) * w + b


def _ln_no_bias(x, w, b, eps):
    return _ORIG["layer_norm"](x, w, np.zeros_like(np.asarray(b, np.float64)), eps)


def _encode_ties_away(v):
    v = np.asarray(v, np.float64)
    out = _ORIG["e4m3_encode"](v)
    pos = okw._POS
    mag = np.minimum(np.abs(v), 448.0)
    hi = np.minimum(np.searchsorted(pos, mag), pos.size - 1)
    tie = (hi > 0) & np.isclose(pos[hi] - mag, mag - pos[np.maximum(hi - 1, 0)], rtol=0, atol=0)
    return np.where(tie, (hi.astype(np.uint8) | (out & 0x80)), out).astype(np.uint8)


def _encode_truncate(v):
    v = np.asarray(v, np.float64)
    mag = np.minimum(np.abs(v), 448.0)
    code = np.maximum(np.searchsorted(okw._POS, mag, side="right") - 1, 0).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def _quantize_wrong_max(y):
    y32 = np.asarray(y, np.float64).astype(np.float32)
    amax = np.abs(y32).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(240.0), np.float32(1.0)).astype(np.float32)
    return _ORIG["e4m3_encode"]((y32 / scale[..., None]).astype(np.float32)), scale


def _slots_off_by_one(ctx_len, block_table, R, num_blocks):
    return _ORIG["write_slots"](np.asarray(ctx_len) + 1, block_table, R, num_blocks)


_ORIG = {name: getattr(okw, name) for name in ("layer_norm", "e4m3_encode", "quantize_rows", "write_slots")}

MUTANTS = {
    "layer_norm_unbiased_variance": ("layer_norm", _ln_unbiased),
    "layer_norm_eps_outside_sqrt": ("layer_norm", _ln_eps_outside),
    "layer_norm_drops_bias": ("layer_norm", _ln_no_bias),
    "e4m3_ties_away_from_zero": ("e4m3_encode", _encode_ties_away),
    "e4m3_truncates": ("e4m3_encode", _encode_truncate),
    "quantize_to_240": ("quantize_rows", _quantize_wrong_max),
    "slots_one_position_late": ("write_slots", _slots_off_by_one),
}

PIN_TESTS = [
    test_layer_norm_matches_torch,
    test_layer_norm_closed_forms,
    test_e4m3_encode_matches_torch_on_values_and_midpoints,
    test_quantize_rows_matches_the_workloads_quantiser,
    test_quantized_row_reaches_the_end_of_the_range_and_stays_close,
    test_write_slots_hand_example,
    test_index_key_write_hand_example,
]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches_the_key_write_mutant(mutant, monkeypatch):
    fname, fn = MUTANTS[mutant]
    monkeypatch.setattr(okw, fname, fn)
    monkeypatch.setattr(oracle, fname, fn)
    caught = []
    for test in PIN_TESTS:
        try:
            test()
        except (AssertionError, IndexError, ValueError):
            caught.append(test.__name__)
    assert caught, f"no pin caught mutant {mutant}"
