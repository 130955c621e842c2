"""CPU oracle for long-context prefill attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 numpy statement of what the GPU library computes.  It is
used by the tests, by the package's smoke check and by the benchmark's CPU
baseline leg, and by nothing else: the library itself never imports, links or
calls anything here, and nothing here imports the library.  Inputs are the same
bf16/fp16 values the GPU receives, widened exactly to float64.

Modules
-------
dense        chunked prefill attention under an additive mask, with the full
             masked score matrix materialised (per head, in row slabs).
blocksparse  mean-pooled key index, alpha-threshold block selection plus the
             local diagonal, and exact-plus-pooled block-sparse attention.

Every function is pinned by ``tests/test_oracle_*.py`` against brute force,
closed forms, library routines or invariants that the method fixes.
"""
from .dense import attention_weights, bits_mask_ref, causal_kmask_ref, dense_ref, fold_mask_ref  # noqa: F401
from .blocksparse import (  # noqa: F401
    pooled_index_ref, selection_votes_ref, select_ref, blocksparse_ref, selection_sets, rule_blocks,
)
