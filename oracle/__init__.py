"""fp64 CPU oracle of the HySparse2 attention hot path (test infrastructure only).

Only the tests, the smoke check of the package entry file and the benchmark's
CPU-baseline leg may import this package. The GPU library does not use it.
"""
from .hs2_oracle import (  # noqa: F401
    attended_rows,
    block_query,
    bridge_kv,
    bridge_kv_fp8,
    candidate_count,
    dequantize_kv,
    e4m3_decode,
    e4m3_encode,
    full_attention,
    logits,
    select_topk,
    selection_scores,
    selector_query,
    sparse_attention,
    window_rows,
)
