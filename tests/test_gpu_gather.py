"""GPU parity of the gather entry (attention over an indexer's compacted
selection, kept keys only) against the fp64 oracle: dense attention under the
mask that the oracle folds from the same lists.

Bar: |gpu - oracle| <= 2e-3 + 1e-2 |oracle| elementwise, as for the dense path
(the gather path keeps scores, weights and sums in fp32, so it sits far inside).
"""
import sys

import numpy as np
import pytest

from oracle import dense_ref, fold_mask_ref
from workloads import bf16_bits, make_workload
from _util import assert_close, dev_bf16, f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lp():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_prefill_attn_amd as m
    m.lib()
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rand_bits(rng, *shape, s=1.0):
    return bf16_bits(rng.standard_normal(shape).astype(np.float32) * s)


def fold2k5_lists(w, q_start, C):
    """The fold2k5 selection of rows q_start .. q_start+C-1 as lists: rows within
    the budget keep every block up to their position, later rows their drawn blocks."""
    s = w.spec
    rows = [list(range(p // s.fold_width + 1)) if p + 1 <= s.fold_budget
            else [int(c) for c in w.keep_blocks[p]] for p in range(q_start, q_start + C)]
    idx = np.zeros((C, max(len(r) for r in rows)), dtype=np.int32)
    for i, r in enumerate(rows):
        idx[i, :len(r)] = r
    return idx, np.array([len(r) for r in rows], dtype=np.int32)


def run_gather(lp, q, k, v, idx, cnt, q_start, width, recent, scale):
    O = lp.prefill_attn_gather(dev_bf16(q), dev_bf16(k), dev_bf16(v), torch.from_numpy(idx).cuda(),
                               torch.from_numpy(cnt).cuda(), q_start, width, recent, scale)
    torch.cuda.synchronize()
    return O.cpu().numpy()


def test_gather_fold2k5(lp):
    """Every chunk of the folded-selection prompt, all heads."""
    w = make_workload("fold2k5")
    s = w.spec
    for q0, C in s.chunks:
        T = q0 + C
        idx, cnt = fold2k5_lists(w, q0, C)
        say("gather fold2k5", q0, C)
        got = run_gather(lp, w.Q[q0:T], w.K[:T], w.V[:T], idx, cnt, q0, s.fold_width, s.fold_recent, s.scale)
        mask = fold_mask_ref(idx, cnt, q0, T, s.fold_width, s.fold_recent)
        want = dense_ref(f64(w.Q[q0:T]), f64(w.K[:T]), f64(w.V[:T]), mask, s.scale)
        say("worst err/bound", assert_close(got, want, f"gather fold2k5 chunk {q0}"))


@pytest.mark.parametrize("C,q_start,T,n_q,n_kv,d,width,recent,K,seed", [
    (300, 500, 900, 4, 2, 128, 8, 5, 40, 41),     # out-of-range, duplicate and negative entries
    (200, 0, 200, 8, 2, 64, 1, 0, 64, 42),        # width 1, no recent keys, d 64, group 4
    (130, 70, 200, 2, 2, 128, 64, 17, 6, 43),     # width 64 (blocks reach past the row)
    (96, 4000, 4096, 6, 3, 128, 4, 3, 300, 44),   # odd group (2), long lists
])
def test_gather_malformed_and_shapes(lp, C, q_start, T, n_q, n_kv, d, width, recent, K, seed):
    rng = np.random.default_rng(seed)
    q, k, v = rand_bits(rng, C, n_q, d), rand_bits(rng, T, n_kv, d), rand_bits(rng, T, n_kv, d)
    idx = rng.integers(-5, T // width + 10, size=(C, K)).astype(np.int32)
    idx[:, 1::7] = idx[:, 0:1]                                 # duplicates within a row
    cnt = rng.integers(-3, K + 20, size=C).astype(np.int32)   # negative and past the list width
    cnt[:3] = 0                                               # rows keeping only their recent keys
    say("gather malformed", C, q_start, T, n_q, n_kv, d, width, recent, K)
    scale = 1.0 / np.sqrt(d)
    got = run_gather(lp, q, k, v, idx, cnt, q_start, width, recent, scale)
    mask = fold_mask_ref(idx, cnt, q_start, T, width, recent)
    want = dense_ref(f64(q), f64(k), f64(v), mask, scale)
    say("worst err/bound", assert_close(got, want, "gather malformed"))
    if recent == 0:
        empty = np.all(mask <= -30000, axis=1)                # rows that keep no key at all
        assert empty[:3].all() and np.all(got[empty] == 0.0)


def test_gather_no_lists(lp):
    """keep_ld 0 (no list array): every row keeps only its recent keys."""
    rng = np.random.default_rng(45)
    C, q_start, T, n_q, n_kv, d, recent = 64, 30, 94, 2, 1, 128, 7
    q, k, v = rand_bits(rng, C, n_q, d), rand_bits(rng, T, n_kv, d), rand_bits(rng, T, n_kv, d)
    idx = np.zeros((C, 0), dtype=np.int32)
    cnt = np.full(C, 5, dtype=np.int32)                       # clamped to the (empty) list width
    say("gather no lists")
    got = run_gather(lp, q, k, v, idx, cnt, q_start, 4, recent, 0.1)
    mask = fold_mask_ref(idx, cnt, q_start, T, 4, recent)
    assert_close(got, dense_ref(f64(q), f64(k), f64(v), mask, 0.1), "gather no lists")


def test_gather_long_history_sampled(lp):
    """A 256-row chunk at the end of a 32K history, each row keeping 512 drawn
    4-key blocks and its 3 most recent keys (the folded selection's shape at long
    context); sampled rows, all heads, against the oracle."""
    rng = np.random.default_rng(46)
    C, T, n_q, n_kv, d = 256, 32768, 16, 8, 128
    q0 = T - C
    q, k, v = rand_bits(rng, C, n_q, d), rand_bits(rng, T, n_kv, d), rand_bits(rng, T, n_kv, d)
    idx = np.stack([rng.choice((q0 + i - 2) // 4, size=512, replace=False) for i in range(C)]).astype(np.int32)
    cnt = np.full(C, 512, dtype=np.int32)
    say("gather 32K history")
    got = run_gather(lp, q, k, v, idx, cnt, q0, 4, 3, 1.0 / np.sqrt(d))
    rows = np.array([0, 1, 77, 128, 200, 255])
    mask = fold_mask_ref(idx[rows], cnt[rows], 0, T, 4, 3)     # rows' own positions below
    for r_i, r in enumerate(rows):
        mask[r_i] = fold_mask_ref(idx[r:r + 1], cnt[r:r + 1], q0 + r, T, 4, 3)[0]
    want = dense_ref(f64(q[rows]), f64(k), f64(v), mask, 1.0 / np.sqrt(d))
    say("worst err/bound", assert_close(got[rows], want, "gather 32K history"))


def test_gather_is_deterministic(lp):
    w = make_workload("fold2k5")
    s = w.spec
    q0, C = s.chunks[-1]
    T = q0 + C
    idx, cnt = fold2k5_lists(w, q0, C)
    a = run_gather(lp, w.Q[q0:T], w.K[:T], w.V[:T], idx, cnt, q0, s.fold_width, s.fold_recent, s.scale)
    b = run_gather(lp, w.Q[q0:T], w.K[:T], w.V[:T], idx, cnt, q0, s.fold_width, s.fold_recent, s.scale)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
