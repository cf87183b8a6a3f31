"""CPU oracle of the sparse-attention decode path. TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg use it; the
HIP library never imports, links or calls anything here.
"""

from . import dsa_oracle  # noqa: F401
from .dsa_oracle import (  # noqa: F401
    bf16_to_f64,
    decode,
    e4m3fn_encode,
    expand_pages,
    e4m3fn_table,
    glm52_indexer_pattern,
    indexer_owner_layers,
    indexer_scores,
    indexer_scores_row,
    kv_append,
    page_budget_select,
    page_scores_row,
    quantize_key_e4m3,
    row_positions,
    run,
    sparse_mla,
    sparse_mla_row,
    topk,
    topk_row,
)
