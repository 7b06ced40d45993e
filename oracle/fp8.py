"""OCP 8-bit floating point, E4M3 variant ("E4M3FN"), decoded from its bit fields.

The pages store index keys and latent rows as FP8 without naming the variant;
the workloads name e4m3, and gfx950 parts use the OCP encoding. Bit layout:
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits. There are no
infinities; exponent 1111 with mantissa 111 is NaN, so the largest finite
magnitude is 1.75 * 2^8 = 448. Exponent 0000 encodes subnormals m/8 * 2^-6.
"""

import numpy as np


def e4m3_value(code: int) -> float:
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """float64 [256]: value of every E4M3 code."""
    return _TABLE.copy()


def e4m3_decode(codes) -> np.ndarray:
    """Decode an array of uint8 E4M3 codes to float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]
