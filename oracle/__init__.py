"""Float64 CPU oracle for the DSA hot path -- test infrastructure only.

Importable from ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg; never from the product path.
"""
from .dsa import (alignment_loss_rows, attention_target_row, bf16_bits_to_f64, dequantize,
                  e4m3fn_decode, forward_rows, indexer_backward_row, indexer_backward_rows,
                  indexer_kl_row, indexer_row, indexer_scores, mha_attention_row, mha_attention_rows,
                  sparse_attention_row, topk_select)

__all__ = ["alignment_loss_rows", "attention_target_row", "bf16_bits_to_f64", "dequantize",
           "e4m3fn_decode", "forward_rows", "indexer_backward_row", "indexer_backward_rows",
           "indexer_kl_row", "indexer_row", "indexer_scores", "mha_attention_row", "mha_attention_rows",
           "sparse_attention_row", "topk_select"]
