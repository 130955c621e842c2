"""The benchmark's work accounting (host arithmetic only, no GPU): the exact
work of a block-sparse call counted by bench.exact_pairs equals a brute-force
count over (row, key) pairs and pooled rows, and with every block kept it equals
the dense causal pair count."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import dense_equiv_pairs  # noqa: E402


def brute_pairs(cnt, q0, C, B):
    """Per KV head and query block j: each row p of the call in block j computes
    its visible keys in the c - 1 kept blocks below j (all B keys), the keys
    j B .. p of the diagonal, and one pooled row per skipped block below j."""
    total = 0
    for g in range(cnt.shape[0]):
        for jj in range(cnt.shape[1]):
            j = q0 // B + jj
            c = int(cnt[g, jj])
            for p in range(max(j * B, q0), min((j + 1) * B, q0 + C)):
                total += (c - 1) * B + (p - j * B + 1) + (j - (c - 1))
    return total


def test_exact_pairs_matches_brute_force():
    rng = np.random.default_rng(5)
    B = 16
    for q0, C in [(0, 100), (37, 90), (64, 64), (200, 1)]:
        j0, j1 = q0 // B, (q0 + C - 1) // B
        cnt = np.array([[rng.integers(1, j + 2) for j in range(j0, j1 + 1)] for _ in range(3)], dtype=np.int32)
        assert bench.exact_pairs(cnt, q0, C, B) == brute_pairs(cnt, q0, C, B), (q0, C)


def test_exact_pairs_all_kept_is_dense():
    B, n_kv = 128, 2
    for q0, C in [(0, 1024), (4096, 4096), (300, 777)]:
        j0, j1 = q0 // B, (q0 + C - 1) // B
        cnt = np.tile(np.arange(j0, j1 + 1, dtype=np.int32) + 1, (n_kv, 1))
        assert bench.exact_pairs(cnt, q0, C, B) == n_kv * dense_equiv_pairs(q0, C)
