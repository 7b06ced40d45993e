"""Index-key write step -- TEST INFRASTRUCTURE ONLY (see the package docstring).

"TokenSpeed Kimi K3.1", section "Integrating sparse attention with the K3
stack", step 1: one fused kernel normalises the new token's index key,
quantises it to FP8 with a single scale and writes it into the cache; the
loader accepts LayerNorm as the only key normalisation (same section).

Readings (the pages give no formula or constants):
* LayerNorm over the 128 dims of one token's key, biased variance (divide by
  128), elementwise affine weight and bias, epsilon supplied by the caller;
* the single scale is the row's absmax over 448 (1 for an all-zero row) and
  the codes are OCP E4M3 (E4M3FN) by round-to-nearest-even, saturating at
  +-448 -- the same reading the workloads use for every stored key;
* the normalisation is computed in float64 here. The quantisation decision
  (which E4M3 code) is taken in float32 like the kernel's: the float64
  output is rounded to float32, the scale is a float32 division and so is
  value / scale. Codes that fall within rounding of an E4M3 midpoint may
  legitimately differ between two correct implementations; the parity tests
  accept either neighbour there.
"""

import numpy as np

from .fp8 import e4m3_table

E4M3_MAX = 448.0

# finite non-negative E4M3 values in code order (codes 0x00 .. 0x7E)
_POS = e4m3_table()[:0x7F]


def layer_norm(x, weight, bias, eps):
    """float64 LayerNorm of each row of x over its last dim."""
    x = np.asarray(x, np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + float(eps)) * np.asarray(weight, np.float64) + np.asarray(bias, np.float64)


def e4m3_encode(v):
    """OCP E4M3 codes of float values: nearest finite value, ties to the even
    code (even mantissa), magnitudes past 448 saturate; the sign of -0 and
    of values that round to zero is kept."""
    v = np.asarray(v, np.float64)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_POS, mag, side="left")  # first value >= mag
    hi = np.minimum(hi, _POS.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS[lo]
    d_hi = _POS[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(mag == _POS[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    neg = np.signbit(v)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def quantize_rows(y):
    """Per-row absmax E4M3 quantisation, decisions in float32.

    Returns (uint8 codes [..., 128], float32 scales [...])."""
    y32 = np.asarray(y, np.float64).astype(np.float32)
    amax = np.abs(y32).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    v = (y32 / scale[..., None]).astype(np.float32)
    return e4m3_encode(v), scale


def index_key_write(k, weight, bias, eps):
    """Codes and scales of new index keys k [rows, 128] (any float dtype)."""
    return quantize_rows(layer_norm(k, weight, bias, eps))


def scatter_rows(codes_plane, scale_plane, codes, scales, slots):
    """Write rows into paged planes ([blocks, 64, 128] and [blocks, 64]) at
    flat cache slots (block * 64 + offset); slots < 0 are skipped. Returns new
    planes (the inputs are not modified)."""
    cp = np.array(codes_plane, copy=True)
    sp = np.array(scale_plane, copy=True)
    for row, slot in enumerate(np.asarray(slots).tolist()):
        if slot < 0:
            continue
        cp[slot // 64, slot % 64] = codes[row]
        sp[slot // 64, slot % 64] = scales[row]
    return cp, sp


def write_slots(ctx_len, block_table, R, num_blocks):
    """Flat cache slot of each new row (request b, row r at position
    ctx_len[b] - R + r), or -1 where the position or its page is invalid."""
    ctx_len = np.asarray(ctx_len, np.int64)
    table = np.asarray(block_table, np.int64)
    out = []
    for b in range(ctx_len.size):
        for r in range(R):
            pos = int(ctx_len[b]) - R + r
            if pos < 0 or pos // 64 >= table.shape[1]:
                out.append(-1)
                continue
            blk = int(table[b, pos // 64])
            out.append(blk * 64 + pos % 64 if 0 <= blk < num_blocks else -1)
    return np.asarray(out, np.int64)
