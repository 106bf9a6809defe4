"""fp64 CPU oracle for dynamic sparse prefill attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or tables); the two meet only in the
seeded inputs of the ``synth`` module.

The oracle is written for readability, not speed: numpy in float64, one rule
per function, each citing the passage it follows.  Pages cited:

  [MInf]   "MInference 1.0: Accelerating Pre-filling for Long-Context LLMs via
           Dynamic Sparse Attention", explainer (abeam.tech) and the authors'
           abstract (zhuanzhiai.com).
  [MoBA]   "Optimizing Mixture of Block Attention" explainer (lifetechia.com).
  [FP]     "FlashPrefill: Instantaneous Pattern Discovery and Thresholding for
           Ultra-Fast Long-Context Prefilling" (gist.science 2603.06199).
  [MISA]   "MISA: Mixture of Indexer Sparse Attention for Long-Context LLM
           Inference" (gist.science 2605.07363).

Parity status: every function is pinned by a test in ``tests/test_oracle.py``
against brute force, a closed form or a library routine, except the choices
the pages leave open (router aggregation, forced blocks with the threshold
rule, indexer key sharing, the two stages of the hierarchical indexer, the
rule that turns pooled block scores into vertical and slash sets); those
are "parity unpinned" beyond brute force of the chosen definition, as stated
in their docstrings.
"""
from .bf16 import round_bf16, to_f64
from .rules import (
    block_means, block_scores, topk_rule, threshold_rule, select_blocks,
    vs_scores, vs_select, ashape_sets,
    mask_dense, mask_vs, mask_block, mask_tokens,
    row_set_vs, row_set_block, row_set_dense,
)
from .attention import masked_attention, attention_rows
from .indexer import indexer_scores, router_heads, token_topk, indexer_row, hierarchical_tokens
from .work import selected_count_vs, selected_count_block, selected_count_dense
from .discovery import pooled_vs_scores, pooled_vs_blocks, expand_blocks, pooled_vs_sets

__all__ = [
    "round_bf16", "to_f64",
    "block_means", "block_scores", "topk_rule", "threshold_rule", "select_blocks",
    "vs_scores", "vs_select", "ashape_sets",
    "mask_dense", "mask_vs", "mask_block", "mask_tokens",
    "row_set_vs", "row_set_block", "row_set_dense",
    "masked_attention", "attention_rows",
    "indexer_scores", "router_heads", "token_topk", "indexer_row", "hierarchical_tokens",
    "selected_count_vs", "selected_count_block", "selected_count_dense",
    "pooled_vs_scores", "pooled_vs_blocks", "expand_blocks", "pooled_vs_sets",
]
