"""Pins of the MXFP4 index-key oracle (E2M1 codes with E8M0 block scales)
against facts that do not come from it: the format's own definition written
out bit by bit, closed forms, the pages' byte counts, round trips of exactly
representable blocks, the rounding error bound, and agreement of MXFP4 and
FP8 scoring on keys both formats hold exactly; plus the mutants they catch.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.dsa as odsa
import oracle.mxfp4 as omx
from workloads import make_case

RNG = np.random.default_rng(20260202)


def _e2m1_from_bits(code):
    """Value of a 4-bit E2M1 code from its fields: sign, 2-bit exponent with
    bias 1, 1-bit mantissa (exponent 0: subnormal, 0.5 * mantissa)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + 0.5 * m)
    return -mag if s else mag


def test_e2m1_table_is_the_format_definition():
    tab = oracle.e2m1_table()
    assert tab.shape == (16,)
    for c in range(16):
        assert tab[c] == _e2m1_from_bits(c) and np.signbit(tab[c]) == bool(c & 8)


def test_key_bytes_match_the_pages():
    # 68 bytes including scales against 132 in FP8: 48.5% less index cache
    assert omx.KEY_BYTES_MXFP4 == 68 and omx.KEY_BYTES_FP8 == 132
    assert round(100 * (1 - omx.KEY_BYTES_MXFP4 / omx.KEY_BYTES_FP8), 1) == 48.5


def test_decode_closed_forms():
    codes = np.zeros((1, 64), np.uint8)
    codes[0, 0] = 0x21  # dim 0: code 1 (0.5), dim 1: code 2 (1.0)
    codes[0, 1] = 0xF7  # dim 2: code 7 (6), dim 3: code 15 (-6)
    y = oracle.mxfp4_decode(codes, np.full((1, 4), 127, np.uint8))[0]
    assert y[:4].tolist() == [0.5, 1.0, 6.0, -6.0] and not y[4:].any()
    # every block has its own power of two: all codes 2 (1.0), scales 2^-1, 2^0, 2^1, 2^3
    y = oracle.mxfp4_decode(np.full((1, 64), 0x22, np.uint8), np.array([[126, 127, 128, 130]], np.uint8))[0]
    assert y.tolist() == [0.5] * 32 + [1.0] * 32 + [2.0] * 32 + [8.0] * 32


def test_encode_closed_forms():
    x = np.concatenate([np.full(32, 6.0), np.full(32, 0.75), np.full(32, -3.0), np.zeros(32)])[None]
    codes, scales = oracle.mxfp4_encode(x)
    # 6 = 6 * 2^0; 0.75 -> floor(log2 0.75) - 2 = -3: 0.75 * 8 = 6; 3 -> exponent -1: 3 * 2 = 6; zeros: byte 127
    assert scales.tolist() == [[127, 124, 126, 127]]
    assert np.array_equal(oracle.mxfp4_decode(codes, scales), x)
    # saturation: 7 in a block whose max is 7 (exponent 0) becomes 6; ties go to the even code
    x = np.zeros((1, 128))
    x[0, 0], x[0, 1], x[0, 2], x[0, 3] = 7.0, 2.5, 5.0, 0.25
    y = oracle.mxfp4_decode(*oracle.mxfp4_encode(x))[0]
    assert y[:4].tolist() == [6.0, 2.0, 4.0, 0.0]


def test_representable_blocks_round_trip_exactly():
    pos = oracle.e2m1_table()
    for _ in range(200):
        k = RNG.integers(-20, 20, size=4)
        vals = pos[RNG.integers(0, 16, size=128)] * np.repeat(np.exp2(k), 32)
        y = oracle.mxfp4_decode(*oracle.mxfp4_encode(vals[None]))[0]
        assert np.array_equal(y, vals)


def test_encode_error_bound():
    x = RNG.standard_normal((500, 128)) * RNG.choice([1e-3, 1.0, 40.0], size=(500, 1))
    codes, scales = oracle.mxfp4_encode(x)
    y = oracle.mxfp4_decode(codes, scales)
    unit = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=-1)
    mag = np.abs(x) / unit
    # half the gap between neighbouring magnitudes, or the overshoot past 6
    half_gap = np.where(mag < 2, 0.25, np.where(mag < 4, 0.5, 1.0))
    bound = np.where(mag > 6, mag - 6, half_gap) * unit
    assert np.all(np.abs(y - x) <= bound * (1 + 1e-12))
    # the largest magnitude of each block lands in [4, 8) after scaling
    blk = mag.reshape(500, 4, 32).max(axis=-1)
    assert np.all((blk >= 4) & (blk < 8))


def _twin_cases():
    """An MXFP4 case and an FP8 case holding the same dequantised keys (E2M1
    values times 2^k with |k| small are exact in E4M3 with scale 1)."""
    f4 = make_case(2, 3, [200, 130], seed=41, key_format="mxfp4", permute_blocks=True)
    f8 = make_case(2, 3, [200, 130], seed=41, permute_blocks=True)
    keys = oracle.mxfp4_decode(f4.key_fp4.numpy(), f4.key_e8m0.numpy())  # [nb, 64, 128]
    codes = torch.tensor(keys, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    assert np.array_equal(oracle.e4m3_decode(codes.numpy()), keys)  # exact in E4M3
    f8.key_fp8 = codes
    f8.key_scale = torch.ones_like(f8.key_scale)
    f8.block_table = f4.block_table.clone()
    f8.q_idx, f8.w = f4.q_idx, f4.w
    return f4, f8


def test_mxfp4_scores_equal_fp8_scores_on_twin_keys():
    f4, f8 = _twin_cases()
    for row in range(f4.rows):
        assert np.array_equal(oracle.row_scores(f4, row), oracle.row_scores(f8, row))


def test_mxfp4_row_scores_by_hand():
    f4 = make_case(1, 2, [70], seed=42, key_format="mxfp4", permute_blocks=True)
    table = f4.block_table[0].numpy()
    row = 1  # position 69: sees tokens 0..69
    pos = np.arange(70)
    codes = f4.key_fp4.numpy()[table[pos // 64], pos % 64]
    scl = f4.key_e8m0.numpy()[table[pos // 64], pos % 64]
    keys = np.zeros((70, 128))
    for t in range(70):
        for d in range(128):
            nib = (codes[t, d // 2] >> (4 * (d % 2))) & 15
            keys[t, d] = _e2m1_from_bits(int(nib)) * 2.0 ** (int(scl[t, d // 32]) - 127)
    q = f4.q_idx.float().numpy()[row].astype(np.float64)
    w = f4.w.float().numpy()[row].astype(np.float64)
    want = np.array([sum(w[h] * max(0.0, float(q[h] @ keys[t])) for h in range(32)) for t in range(70)])
    assert np.allclose(oracle.row_scores(f4, row), want, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- mutants

_ORIG = {n: getattr(omx, n) for n in ("mxfp4_decode", "mxfp4_encode", "e2m1_table")}


def _decode_swapped_nibbles(codes, scales):
    c = np.asarray(codes, np.uint8)
    return _ORIG["mxfp4_decode"](((c & 15) << 4) | (c >> 4), scales)


def _decode_bias_126(codes, scales):
    return _ORIG["mxfp4_decode"](codes, np.asarray(scales, np.int64) + 1)


def _decode_block_16(codes, scales):
    c = np.asarray(codes, np.uint8)
    s = np.asarray(scales, np.uint8)
    out = _ORIG["mxfp4_decode"](c, s)
    unit32 = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=-1)
    unit16 = np.repeat(np.exp2(np.repeat(s, 2, axis=-1)[..., :4].astype(np.float64) - 127), 32, axis=-1)
    return out / unit32 * unit16


def _encode_emax_1(x):
    """Block exponent floor(log2 amax) - 1: the largest value lands in [2, 4)."""
    x = np.asarray(x, np.float64)
    blocks = x.reshape(*x.shape[:-1], -1, 32)
    amax = np.abs(blocks).max(axis=-1)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 1, 0).astype(np.int64)
    scaled = blocks / np.exp2(e)[..., None]
    mag = omx._e2m1_round(np.abs(scaled))
    code = np.where(np.signbit(scaled), mag | 8, mag).astype(np.uint8).reshape(x.shape)
    return (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8), (e + 127).astype(np.uint8)


def _table_subnormal_one():
    t = _ORIG["e2m1_table"]().copy()
    t[1], t[9] = 1.0, -1.0
    return t


MUTANTS = {
    "nibbles_swapped": ("mxfp4_decode", _decode_swapped_nibbles),
    "scale_bias_126": ("mxfp4_decode", _decode_bias_126),
    "scale_per_16_values": ("mxfp4_decode", _decode_block_16),
    "encode_exponent_off_by_one": ("mxfp4_encode", _encode_emax_1),
    "subnormal_code_is_one": ("e2m1_table", _table_subnormal_one),
}

PIN_TESTS = [
    test_e2m1_table_is_the_format_definition,
    test_decode_closed_forms,
    test_encode_closed_forms,
    test_representable_blocks_round_trip_exactly,
    test_encode_error_bound,
    test_mxfp4_row_scores_by_hand,
]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches_the_mxfp4_mutant(mutant, monkeypatch):
    fname, fn = MUTANTS[mutant]
    monkeypatch.setattr(omx, fname, fn)
    monkeypatch.setattr(oracle, fname, fn)
    if fname == "mxfp4_decode":
        monkeypatch.setattr(odsa, "mxfp4_decode", fn)
    caught = []
    for test in PIN_TESTS:
        try:
            test()
        except (AssertionError, IndexError, ValueError):
            caught.append(test.__name__)
    assert caught, f"no pin caught mutant {mutant}"
