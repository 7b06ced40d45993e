"""MXFP4 index keys -- TEST INFRASTRUCTURE ONLY (see the package docstring).

"vLLM Day-0 Support for Kimi K3.1 Pro", section "Native MXFP4 indexer": an
MXFP4 index key takes 68 bytes including its scales, against 132 in FP8, and
the indexer scores it with native FP4 matrix instructions, fp32 accumulation
and the weighted reduction over heads ("Inside vLLM's hybrid KV cache" lists
the same two widths).

Readings (the pages give the widths, not the format's details):
* MXFP4 is the OCP Microscaling format: blocks of 32 values share one E8M0
  scale 2^(e - 127), each value an E2M1 code (sign, 2 exponent bits with
  bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6). A 128-dim
  key is 64 bytes of codes and 4 scale bytes: 68 bytes;
* two codes per byte, dim 2i in the low nibble of byte i;
* encoding (used to build pins, not by the scoring path): the block's scale
  exponent is floor(log2(max |x|)) - 2 (so that the largest magnitude lands
  in [4, 8) before rounding), values round to the nearest E2M1 magnitude,
  ties to the even code, saturating at 6.
"""

import numpy as np

_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BLOCK = 32


def e2m1_table():
    """float64 [16]: the value of each E2M1 code (bit 3 is the sign)."""
    return np.concatenate([_E2M1_POS, -_E2M1_POS])


def mxfp4_decode(codes, scales):
    """codes uint8 [..., 64] (two E2M1 codes per byte), scales uint8 [..., 4]
    (E8M0) -> float64 [..., 128]."""
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.uint8)
    lo = codes & 0x0F
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    vals = e2m1_table()[nib]
    factor = np.exp2(scales.astype(np.float64) - 127.0)  # [..., 4]
    return vals * np.repeat(factor, BLOCK, axis=-1)


def _e2m1_round(mag):
    """Nearest E2M1 magnitude code (0..7) of |v| (already divided by the
    block scale), ties to the even code, saturating at 6."""
    mag = np.minimum(np.asarray(mag, np.float64), 6.0)
    hi = np.minimum(np.searchsorted(_E2M1_POS, mag, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E2M1_POS[lo]
    d_hi = _E2M1_POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(mag == _E2M1_POS[hi], hi, np.where(pick_hi, hi, lo))


def mxfp4_encode(x):
    """OCP MXFP4 encoding of x [..., 128] -> (codes uint8 [..., 64], scales
    uint8 [..., 4]). An all-zero block gets scale byte 127 and zero codes."""
    x = np.asarray(x, np.float64)
    blocks = x.reshape(*x.shape[:-1], x.shape[-1] // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0).astype(np.int64)
    e = np.clip(e, -127, 127)
    scaled = blocks / np.exp2(e)[..., None]
    mag_code = _e2m1_round(np.abs(scaled))
    code = np.where(np.signbit(scaled), mag_code | 8, mag_code).astype(np.uint8)
    code = code.reshape(*x.shape[:-1], x.shape[-1])
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


KEY_BYTES_MXFP4 = 128 // 2 + 128 // BLOCK  # 64 code bytes + 4 scale bytes
KEY_BYTES_FP8 = 128 + 4  # 128 E4M3 codes + one fp32 scale
