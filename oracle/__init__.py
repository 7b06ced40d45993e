"""Oracle for the DSA decode/prefill hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, float64 CPU restatement of what Kimi K3.1 Pro's sparse layer
computes, written from the pages' description of the method:

* score: every query row's 32 indexer heads score one FP8 index key per
  earlier token, combined as sum_h w_h * ReLU(q_h . k_s * scale_s)
  (the DeepSeek-V3.2 form that "vLLM Day-0 Support for Kimi K3.1 Pro",
  section "What Kimi K3.1 Pro changes", points to);
* select: the 2,048 highest-scoring positions per row ("TokenSpeed Kimi
  K3.1", section "Integrating sparse attention with the K3 stack", step 3);
* attend: exact softmax attention over only the selected 576-wide latent
  rows, values from their first 512 dims (same section, step 4; "Kimi K3.1
  Pro on AMD Instinct", model overview).

It shares no code with the HIP library and imports nothing from it. Only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package; the product path never does.

Parity status of each function (see the pins in tests/test_oracle_pins.py):
e4m3_table, gather_tokens, index_scores, topk_positions, attend, dsa_rows and
dsa_bytes are pinned against closed forms, library routines or the pages'
printed numbers; key_write's layer_norm, e4m3_encode, quantize_rows and
write_slots against torch's layer_norm and float8 cast, closed forms and the
workloads' own quantiser.
"""

from .fp8 import e4m3_table, e4m3_decode  # noqa: F401
from .dsa import (  # noqa: F401
    attend,
    dense_attend_row,
    dequant,
    dsa_rows,
    gather_tokens,
    index_scores,
    row_scores,
    topk_positions,
)
from .traffic import dsa_bytes, dense_mla_bytes, counted_bytes  # noqa: F401
from .mxfp4 import e2m1_table, mxfp4_decode, mxfp4_encode  # noqa: F401
from .dcp import dcp_select, local_topk, lse_combine, shard_attend  # noqa: F401
from .key_write import (  # noqa: F401
    e4m3_encode,
    index_key_write,
    layer_norm,
    quantize_rows,
    scatter_rows,
    write_slots,
)
