"""Pins for the block-sparse oracle (pooled index, selection, exact-plus-pooled attention).

Independent checks: exact rational / 50-digit brute force, numpy's mean, torch
SDPA in fp64, closed forms and the limits the method fixes (alpha = 0 keeps
every block, alpha >= 1 keeps only the diagonal).
"""
import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

from oracle import (blocksparse_ref, dense_ref, pooled_index_ref, select_ref,
                    selection_sets, selection_votes_ref)
from oracle.blocksparse import pooled_scores
from workloads import bf16_bits, bf16_to_f32, causal_mask, make_workload


def _bf16(rng, *shape, scale=1.0):
    return bf16_to_f32(bf16_bits(rng.standard_normal(shape) * scale)).astype(np.float64)


# ---------------------------------------------------------------- pooled index
def test_pooled_index_matches_numpy_mean_within_one_ulp():
    rng = np.random.default_rng(0)
    T, Hkv, d, B = 1000, 3, 16, 128            # 7 full blocks and a partial one
    K, V = _bf16(rng, T, Hkv, d), _bf16(rng, T, Hkv, d)
    kp, vp = pooled_index_ref(K, V, B)
    assert kp.shape == (Hkv, 8, d) and kp.dtype == np.float32
    for X, P in ((K, kp), (V, vp)):
        for b in range(8):
            want = X[b * B:min((b + 1) * B, T)].mean(axis=0).astype(np.float32)   # [Hkv][d]
            ulp = np.spacing(np.abs(want))
            assert np.all(np.abs(P[:, b, :] - want) <= ulp)


def test_pooled_index_closed_form_arithmetic_sequence():
    # key t holds 0.5*t in every slot: the mean of block [t0, t1) is 0.25*(t0+t1-1)
    T, B = 300, 64
    K = np.repeat((0.5 * np.arange(T))[:, None, None], 4, axis=2)
    kp, vp = pooled_index_ref(K, -K, B)
    for b in range(5):
        t0, t1 = b * B, min((b + 1) * B, T)
        assert np.all(kp[0, b] == np.float32(0.25 * (t0 + t1 - 1)))
        assert np.all(vp[0, b] == np.float32(-0.25 * (t0 + t1 - 1)))


def test_pooling_toy_count():
    """A 6-query x 6-key toy block needs 36 dot products exactly and 6 against
    the pooled key ("Porting FlashPrefill V2", Compress keys before the heavy work)."""
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((6, 4)), rng.standard_normal((6, 1, 4))
    kp, _ = pooled_index_ref(k, k, 6)
    assert (q @ k[:, 0, :].T).size == 36
    assert pooled_scores(q, kp[0]).size == 6


# ---------------------------------------------------------------- selection
def _brute_sets(Q, Kp, q_start, B, alpha, scale):
    """Exact rational scores, weight-space test exp(scale*(r_b - M)) > alpha at 60 digits."""
    mpmath.mp.dps = 60
    C, Hq, d = Q.shape
    Hkv = Kp.shape[0]
    group = Hq // Hkv
    a = mpmath.mpf(float(np.float32(alpha)))
    s = mpmath.mpf(float(np.float32(scale)))
    out = {}
    for g in range(Hkv):
        for j in range(q_start // B, (q_start + C - 1) // B + 1):
            kept = set()
            for h in range(g * group, (g + 1) * group):
                for p in range(max(j * B, q_start), min((j + 1) * B, q_start + C)):
                    q = [Fraction(float(x)) for x in Q[p - q_start, h]]
                    r = [sum(qd * Fraction(float(kd)) for qd, kd in zip(q, Kp[g, b])) for b in range(j)]
                    if not r:
                        continue
                    M = max(r)
                    for b, rb in enumerate(r):
                        diff = rb - M
                        w = mpmath.exp(s * mpmath.mpf(diff.numerator) / diff.denominator)
                        if w > a:
                            kept.add(b)
            out[(g, j)] = sorted(kept) + [j]
    return out


@pytest.mark.parametrize("seed,q_start,alpha", [(0, 0, 0.2), (1, 14, 0.1), (2, 37, 0.5)])
def test_selection_matches_exact_bruteforce(seed, q_start, alpha):
    rng = np.random.default_rng(seed)
    B, d, Hq, Hkv, C = 4, 6, 4, 2, 40
    T = q_start + C
    Q = _bf16(rng, C, Hq, d, scale=3.0)
    K = _bf16(rng, T, Hkv, d, scale=3.0)
    kp, _ = pooled_index_ref(K, K, B)
    scale = float(np.float32(1 / math.sqrt(d)))
    got = selection_sets(Q, kp, q_start, B, alpha, scale)
    want = _brute_sets(Q, kp, q_start, B, alpha, scale)
    assert got == want
    # the test is not vacuous: some blocks pruned, some kept beyond the diagonal
    assert any(len(v) > 1 for v in got.values())
    assert sum(len(v) for v in got.values()) < sum(j + 1 for (g, j) in got)


def test_selection_limits_and_monotonicity():
    rng = np.random.default_rng(3)
    B, d, Hq, Hkv, C, q_start = 8, 16, 4, 2, 64, 40
    T = q_start + C
    Q, K = _bf16(rng, C, Hq, d, scale=1.5), _bf16(rng, T, Hkv, d, scale=1.5)
    kp, _ = pooled_index_ref(K, K, B)
    scale = 0.25
    every = selection_sets(Q, kp, q_start, B, 0.0, scale)
    assert all(v == list(range(j + 1)) for (g, j), v in every.items())      # alpha = 0 prunes nothing
    for a in (1.0, 2.0):
        only = selection_sets(Q, kp, q_start, B, a, scale)
        assert all(v == [j] for (g, j), v in only.items())                  # alpha >= 1: diagonal only
    prev = every
    for a in (0.01, 0.05, 0.1, 0.2, 0.5, 0.9):
        cur = selection_sets(Q, kp, q_start, B, a, scale)
        assert all(set(cur[key]) <= set(prev[key]) for key in cur)          # monotone in alpha
        prev = cur
    # for 0 < alpha < 1 each row's hottest block is always voted for
    for i in range(C):
        p = q_start + i
        j = p // B
        if j == 0:
            continue
        votes = selection_votes_ref(Q[i:i + 1, 0], kp[0, :j], 0.3, scale)
        assert votes[0, int(np.argmax(pooled_scores(Q[i:i + 1, 0], kp[0, :j])))]


def test_kept_by_rule_closed_forms():
    """With alpha = 1 no row votes, so the selection is exactly the rule sets plus
    the diagonal (figure "Where the kept blocks are": sinks = the first 256
    tokens, a local window next to the diagonal, the last tiles dense)."""
    rng = np.random.default_rng(8)
    B, d, C, q_start = 128, 16, 3 * 128, 9 * 128         # query blocks 9, 10, 11 over 12 key blocks
    Q = _bf16(rng, C, 2, d)
    kp = _bf16(rng, 1, 12, d).astype(np.float32)
    sets = selection_sets(Q, kp, q_start, B, 1.0, 0.25, sink_tokens=256, window_blocks=3)
    assert sets[(0, 9)] == [0, 1, 6, 7, 8, 9]
    assert sets[(0, 10)] == [0, 1, 7, 8, 9, 10]
    assert sets[(0, 11)] == [0, 1, 8, 9, 10, 11]
    # a sink that is not a whole block keeps the block it starts; the window stops at 0
    assert selection_sets(Q, kp, q_start, B, 1.0, 0.25, sink_tokens=1, window_blocks=20)[(0, 9)] == \
        list(range(10))
    # the last two query blocks of the call attend densely
    tail = selection_sets(Q, kp, q_start, B, 1.0, 0.25, dense_tail_blocks=2)
    assert tail[(0, 9)] == [9] and tail[(0, 10)] == list(range(11)) and tail[(0, 11)] == list(range(12))
    # rules only add: every voted block stays kept
    plain = selection_sets(Q, kp, q_start, B, 0.3, 0.25)
    ruled = selection_sets(Q, kp, q_start, B, 0.3, 0.25, sink_tokens=300, window_blocks=2,
                           dense_tail_blocks=1)
    for key in plain:
        assert set(plain[key]) <= set(ruled[key])


def test_select_ref_arrays_layout():
    rng = np.random.default_rng(4)
    B, d, Hq, Hkv, C, q_start = 8, 8, 2, 1, 30, 13
    T = q_start + C
    Q, K = _bf16(rng, C, Hq, d), _bf16(rng, T, Hkv, d)
    kp, _ = pooled_index_ref(K, K, B)
    idx, cnt = select_ref(Q, kp, q_start, B, 0.2, 0.3)
    nb = -(-T // B)
    j0, j1 = q_start // B, (q_start + C - 1) // B
    assert idx.shape == (Hkv, j1 - j0 + 1, nb) and cnt.shape == (Hkv, j1 - j0 + 1)
    for jj in range(j1 - j0 + 1):
        row = idx[0, jj]
        n = cnt[0, jj]
        assert row[n - 1] == j0 + jj                       # diagonal last
        assert np.all(np.diff(row[:n]) > 0)                # strictly ascending
        assert np.all(row[n:] == 0)                        # zero-filled tail


# ---------------------------------------------------------------- attention
def _small_problem(seed, N=300, Hq=4, Hkv=2, d=16, q_start=100, B=32, sc=1.0):
    rng = np.random.default_rng(seed)
    Q = _bf16(rng, N, Hq, d, scale=sc)
    K = _bf16(rng, N, Hkv, d, scale=sc)
    V = _bf16(rng, N, Hkv, d)
    C = N - q_start
    return Q[q_start:], K, V, q_start, C, B


@pytest.mark.parametrize("q_start", [0, 100])
def test_alpha_zero_equals_dense_causal(q_start):
    Q, K, V, q_start, C, B = _small_problem(0, q_start=q_start)
    kp, vp = pooled_index_ref(K, V, B)
    idx, cnt = select_ref(Q, kp, q_start, B, 0.0, 0.25)
    got = blocksparse_ref(Q, K, V, kp, vp, idx, cnt, q_start, B, 0.25)
    want = dense_ref(Q, K, V, causal_mask(q_start, C), 0.25)
    assert np.max(np.abs(got - want)) < 1e-12


def test_blockwise_constant_kv_equals_dense_for_any_alpha():
    """If K and V are constant inside every block, B*exp(q.kbar) equals the sum of
    the block's B exact weights, so pooling loses nothing."""
    rng = np.random.default_rng(6)
    N, Hq, Hkv, d, B, q_start = 320, 4, 2, 16, 32, 64
    nb = N // B
    Kb = _bf16(rng, nb, Hkv, d, scale=1.5)
    Vb = _bf16(rng, nb, Hkv, d)
    K = np.repeat(Kb, B, axis=0)
    V = np.repeat(Vb, B, axis=0)
    Q = _bf16(rng, N - q_start, Hq, d, scale=1.5)
    kp, vp = pooled_index_ref(K, V, B)
    want = dense_ref(Q, K, V, causal_mask(q_start, N - q_start), 0.25)
    for alpha in (0.05, 0.3, 1.0):
        idx, cnt = select_ref(Q, kp, q_start, B, alpha, 0.25)
        assert cnt.sum() < cnt.size * nb                       # something was pruned
        got = blocksparse_ref(Q, K, V, kp, vp, idx, cnt, q_start, B, 0.25)
        assert np.max(np.abs(got - want)) < 1e-12


def test_blocksparse_equals_sdpa_over_augmented_keys():
    """Each row == SDPA over {exact keys} + {pooled keys with additive bias ln B}."""
    Q, K, V, q_start, C, B = _small_problem(7, q_start=37, sc=1.5)
    scale = 0.25
    kp, vp = pooled_index_ref(K, V, B)
    idx, cnt = select_ref(Q, kp, q_start, B, 0.15, scale)
    got = blocksparse_ref(Q, K, V, kp, vp, idx, cnt, q_start, B, scale)
    Hq, Hkv = Q.shape[1], K.shape[1]
    j0 = q_start // B
    for i in range(0, C, 7):
        p = q_start + i
        j = p // B
        for h in range(Hq):
            g = h // (Hq // Hkv)
            kept = set(idx[g, j - j0, :cnt[g, j - j0]].tolist())
            ex = [t for t in range(p + 1) if (t // B) in kept]
            pooled = [b for b in range(j) if b not in kept]
            keys = np.concatenate([K[ex, g], kp[g, pooled].astype(np.float64)])
            vals = np.concatenate([V[ex, g], vp[g, pooled].astype(np.float64)])
            bias = np.concatenate([np.zeros(len(ex)), np.full(len(pooled), math.log(B))])
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(Q[i:i + 1, h][None]), torch.from_numpy(keys[None]),
                torch.from_numpy(vals[None]), attn_mask=torch.from_numpy(bias[None, None]),
                scale=scale)
            assert np.max(np.abs(o.numpy()[0, 0] - got[i, h])) < 1e-12


def _restricted_mask(rows_abs, T, B, kept_of_row):
    m = np.full((len(rows_abs), T), -30000.0)
    for r, p in enumerate(rows_abs):
        for b in kept_of_row(p):
            m[r, b * B:min((b + 1) * B, p + 1)] = 0.0
    return m


def test_planted_workload_controls_are_not_vacuous():
    """Negative controls on the planted 32K workload, on the rows the block-sparse
    GPU test checks, over all KV heads: dropping the pooled correction, and
    block-sparse at alpha 0.1 against dense, must each move some checked output
    by >= 10x the GPU tolerance, and every KV head's checked rows by >= 2x
    (correction) and >= 4x (alpha), so that a GPU path that skipped either part
    would fail parity. (With N(0,1) key noise, mean pooling under-represents a
    skipped block's mass, so the correction moves a row by a few tolerance units
    on most rows; the checked rows include the ones where it moves most.)"""
    from _util import PLANTED32K_ROWS
    w = make_workload("sparse32k")
    s = w.spec
    B, N, grp = s.block, s.N, s.n_q // s.n_kv
    Q = bf16_to_f32(w.Q).astype(np.float64)
    K = bf16_to_f32(w.K).astype(np.float64)
    V = bf16_to_f32(w.V).astype(np.float64)
    kp, vp = pooled_index_ref(K, V, B)
    rows = np.array(PLANTED32K_ROWS)
    qblocks = sorted({int(p) // B for p in rows})
    sets = selection_sets(Q, kp, 0, B, s.alpha, s.scale, qblocks=qblocks)
    nb = N // B
    idx = np.zeros((s.n_kv, nb, nb), dtype=np.int32)
    cnt = np.ones((s.n_kv, nb), dtype=np.int32)
    for (g, j), kept in sets.items():
        idx[g, j, :len(kept)] = kept
        cnt[g, j] = len(kept)
    sparse = blocksparse_ref(Q, K, V, kp, vp, idx, cnt, 0, B, s.scale, rows=rows)
    tol = 2e-3 + 1e-2 * np.abs(sparse)
    corr, alpha = [], []
    for g in range(s.n_kv):
        hs = list(range(g * grp, (g + 1) * grp))
        Qg, Kg, Vg = Q[rows][:, hs], K[:, g:g + 1], V[:, g:g + 1]
        no_corr = dense_ref(Qg, Kg, Vg, _restricted_mask(rows, N, B, lambda p: sets[(g, p // B)]), s.scale)
        dense = dense_ref(Qg, Kg, Vg, _restricted_mask(rows, N, B, lambda p: range(p // B + 1)), s.scale)
        corr.append(float(np.max(np.abs(no_corr - sparse[:, hs]) / tol[:, hs])))
        alpha.append(float(np.max(np.abs(dense - sparse[:, hs]) / tol[:, hs])))
    assert max(corr) >= 10.0 and min(corr) >= 2.0, corr
    assert max(alpha) >= 10.0 and min(alpha) >= 4.0, alpha
    # the selection really is sparse on this workload (about 85% of visible blocks skipped)
    kept = sum(len(v) for v in sets.values())
    assert kept / (s.n_kv * sum(j + 1 for j in qblocks)) < 0.3
