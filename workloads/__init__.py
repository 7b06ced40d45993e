"""Seeded synthetic inputs for the DSA decode and prefill hot path.

This package is shared by the HIP product path, the oracle, the tests and the
benchmark. It only draws random numbers and packs them into the paged-cache
layout; it holds none of the method's arithmetic (no scoring, selection or
attention).
"""

from .gen import (  # noqa: F401
    BLOCK,
    D_IDX,
    D_LAT,
    D_V,
    H_IDX,
    H_MLA,
    TOPK,
    DsaCase,
    case_config,
    make_case,
    quantize_e4m3_rows,
    structure_kwargs,
)
