"""Accounting helpers and the selection rule against figures the pages print
(tests/golden/page_figures.json holds each figure with its source)."""
import json
import math
import os

import numpy as np

from oracle import selection_votes_ref
from workloads import CONFIGS, kv_cache_bytes, score_matrix_bytes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_score_matrix_size():
    g = GOLD["score_matrix_bytes"]
    assert score_matrix_bytes(g["tokens"], g["heads"], g["dtype_bytes"]) > g["at_least"]


def test_kv_cache_formula():
    g = GOLD["kv_cache_bytes"]
    b = kv_cache_bytes(g["n_layers"], g["n_heads"], g["head_dim"], g["seq_len"], g["dtype_bytes"])
    assert round(b / 1e9, 2) == g["approx_gb"]


def test_fold_budget_matches_generator():
    g = GOLD["fold_budget"]
    assert g["kept_blocks"] * g["compress_ratio"] + (g["compress_ratio"] - 1) == g["visible_keys"]
    spec = CONFIGS["fold2k5"]
    assert spec.fold_blocks == g["kept_blocks"] and spec.fold_width == g["compress_ratio"]
    assert spec.fold_budget == g["visible_keys"]


def test_masked_vs_gathered_and_gather_sizing():
    g = GOLD["masked_vs_gathered_scores"]
    assert round(g["chunk"] * g["dense_keys"] / (g["chunk"] * g["gathered_keys"])) == g["approx_ratio"]
    g = GOLD["gather_materialisation"]
    assert round(g["operands"] * g["budget"] * g["head_dim"] / g["total"]) == g["approx_ratio"]


def test_pruned_block_cost_ratio():
    """The page's "128x cheaper per pruned block", through the benchmark's work
    accounting: pruning one visible block of a query block removes B exact keys
    per row and adds one pooled row, so the block costs rows x B when kept and
    rows x 1 when pruned."""
    import bench
    g = GOLD["pruned_block_cost"]
    B = CONFIGS["sparse32k"].block
    assert B == g["block"]
    q0, C = 0, 4 * B                                   # query blocks 0..3, block 3 sees 4 blocks
    kept_all = np.array([[1, 2, 3, 4]], dtype=np.int32)
    pruned = kept_all.copy()
    pruned[0, 3] -= 1                                  # one of block 3's visible blocks pruned
    rows = B
    removed = bench.exact_pairs(kept_all, q0, C, B) - bench.exact_pairs(pruned, q0, C, B)
    kept_cost = rows * B
    pruned_cost = kept_cost - removed
    assert pruned_cost == rows
    assert kept_cost // pruned_cost == g["ratio"]


def test_alpha_toy_selection():
    g = GOLD["alpha_toy"]
    w = np.array(g["relative_weights"])
    scale = 0.5
    # pooled scores r_b with exp(scale * (r_b - max r)) equal to the listed relative weights
    kbar = (np.log(w) / scale)[:, None]
    votes = selection_votes_ref(np.array([[1.0]]), kbar, g["alpha"], scale)
    assert list(np.nonzero(votes[0])[0]) == g["kept"]
