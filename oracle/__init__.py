"""CPU oracle for the CSA/HCA compressed-KV attention step.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or run anything in this package.  The
product path (the HIP library and its Python binding) never calls it, and this
package imports nothing from the product path: the two share no code.  The only
module both sides draw from is `workloads` (seeded inputs, no method arithmetic).

Source of the method: "DeepSeek-V4: Towards Highly Efficient Million-Token
Context Intelligence Review" (dimensionstp.github.io), sections 2-1, 3-2 item 2
(component and config tables) and 3-2 item 4 (indexer QK path, KV-cache layout).
The page gives the structure only; where it is silent the reading taken is
stated at each function.

Pins: every function is checked in tests/test_oracle_*.py against closed forms,
brute force on tiny inputs, exact rational arithmetic, invariants and library
routines (torch scaled_dot_product_attention, torch bf16 conversion), never
against a retyped copy of itself.  No function here is "parity unpinned".
"""
from .csa_hca import (
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    kv_compress,
    n_visible,
    index_scores,
    topk_select,
    index_scores_rows,
    index_scores_fp4_rows,
    topk_select_rows,
    attention,
    csa_query,
    hca_query,
    csa_decode,
    hca_decode,
    hybrid_decode,
    csa_prefill,
    window_tokens,
    attention_union,
    csa_query_swa,
    hca_query_swa,
    attention_sink,
    csa_query_sink,
    hca_query_sink,
    fp4_values,
    fp4_unpack,
    index_scores_fp4,
    csa_query_fp4,
    fp8_e4m3_values,
    kv8_values,
    KV8_ROW_BYTES,
    compress_to_cache,
    fp8_e4m3_round,
    compress_to_cache_kv8,
)

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "kv_compress", "n_visible", "index_scores",
    "topk_select", "index_scores_rows", "index_scores_fp4_rows", "topk_select_rows",
    "attention", "csa_query", "hca_query", "csa_decode", "hca_decode",
    "hybrid_decode", "csa_prefill", "window_tokens", "attention_union", "csa_query_swa",
    "hca_query_swa", "attention_sink", "csa_query_sink", "hca_query_sink",
    "fp4_values", "fp4_unpack", "index_scores_fp4", "csa_query_fp4",
    "fp8_e4m3_values", "kv8_values", "KV8_ROW_BYTES", "compress_to_cache", "fp8_e4m3_round",
    "compress_to_cache_kv8",
]
