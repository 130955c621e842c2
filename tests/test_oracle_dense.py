"""Pins for the dense oracle: brute force, a library routine, closed forms, invariants.

None of these re-types the oracle's formula: each check comes from a different
computation (50-digit mpmath, torch's scaled_dot_product_attention in fp64, or
values fixed by the mathematics).
"""
import math

import mpmath
import numpy as np
import pytest
import torch

from oracle import attention_weights, bits_mask_ref, causal_kmask_ref, dense_ref, fold_mask_ref
from workloads import CONFIGS, bf16_to_f32, causal_mask, dense_equiv_pairs, make_workload

DROP = -30000.0


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _mp_attention(q, k, v, mask, scale):
    """Brute force at 50 digits: omitted keys are skipped, others use exp(s)."""
    mpmath.mp.dps = 50
    C, Hq, d = q.shape
    T, Hkv, _ = k.shape
    group = Hq // Hkv
    out = np.zeros((C, Hq, d))
    for h in range(Hq):
        g = h // group
        for i in range(C):
            terms = []
            for t in range(T):
                if mask[i, t] <= DROP:
                    continue
                dot = mpmath.fsum(mpmath.mpf(float(q[i, h, e])) * mpmath.mpf(float(k[t, g, e]))
                                  for e in range(d))
                terms.append((mpmath.mpf(float(scale)) * dot + mpmath.mpf(float(mask[i, t])), t))
            if not terms:
                continue
            ws = [(mpmath.exp(s), t) for s, t in terms]
            den = mpmath.fsum(w for w, _ in ws)
            for e in range(d):
                num = mpmath.fsum(w * mpmath.mpf(float(v[t, g, e])) for w, t in ws)
                out[i, h, e] = float(num / den)
    return out


def _sdpa(q, k, v, mask, scale):
    """torch SDPA in fp64 on the CPU with dropped keys as -inf and explicit repeat_kv."""
    C, Hq, d = q.shape
    T, Hkv, _ = k.shape
    rep = Hq // Hkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2))).double()
    kt = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2))).double().repeat_interleave(rep, 0)
    vt = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2))).double().repeat_interleave(rep, 0)
    m = torch.from_numpy(np.asarray(mask[:, :T], dtype=np.float64))
    m = torch.where(m <= DROP, torch.tensor(-math.inf, dtype=torch.float64), m)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=float(scale))
    return o.numpy().transpose(1, 0, 2)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dense_matches_mpmath_bruteforce(seed):
    rng = np.random.default_rng(seed)
    C, T, Hq, Hkv, d = 5, 11, 4, 2, 6
    q, k, v = _rand(rng, C, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
    mask = np.where(rng.random((C, T)) < 0.3, DROP, rng.normal(0, 1.5, (C, T)))
    mask[2, :] = DROP                       # an all-dropped row outputs zeros
    mask[3, :] = DROP
    mask[3, 7] = -2.5                       # a single visible key with a bias
    scale = float(np.float32(1 / math.sqrt(d)))
    got = dense_ref(q, k, v, mask, scale)
    want = _mp_attention(q, k, v, mask, scale)
    assert np.max(np.abs(got - want)) < 1e-13
    assert np.all(got[2] == 0.0)


# ---------------------------------------------------------------- library routine
@pytest.mark.parametrize("name", ["tiny", "gqa4k", "fold2k5"])
def test_dense_matches_torch_sdpa_fp64(name):
    w = make_workload(name)
    spec = w.spec
    for idx in range(len(spec.chunks)):
        q_start, C, T, Q, K, V, mask = w.chunk(idx)
        rows = np.arange(C) if C <= 512 else np.linspace(0, C - 1, 384).astype(int)
        q = bf16_to_f32(Q).astype(np.float64)
        k = bf16_to_f32(K).astype(np.float64)
        v = bf16_to_f32(V).astype(np.float64)
        got = dense_ref(q, k, v, mask, spec.scale, rows=rows)
        want = _sdpa(q[rows], k, v, mask[rows], spec.scale)
        assert np.max(np.abs(got - want)) < 1e-12, (name, idx)


# ---------------------------------------------------------------- invariants
def test_softmax_rows_sum_to_one_and_dropped_weights_are_exact_zero():
    rng = np.random.default_rng(7)
    R, T, d = 64, 300, 32
    q, k = _rand(rng, R, d) * 3, _rand(rng, T, d) * 3
    mask = np.where(rng.random((R, T)) < 0.5, DROP, 0.0).astype(np.float16)
    mask[:, 0] = 0  # every row keeps at least one key
    w = attention_weights(q, k, mask, 0.125)
    assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 1e-14
    assert np.all(w[mask <= DROP] == 0.0)
    assert np.all(w[mask > DROP] > 0.0)


def test_mask_is_additive_and_unscaled():
    # two identical keys, biases 0 and ln 3 -> weights exactly 1/4 and 3/4
    q = np.array([[0.7, -1.3]])
    k = np.array([[0.2, 0.5], [0.2, 0.5]])
    mask = np.array([[0.0, math.log(3.0)]])
    w = attention_weights(q, k, mask, 0.37)
    assert np.allclose(w, [[0.25, 0.75]], rtol=0, atol=1e-15)


def test_masked_equals_gathered():
    """Omitting keys through the mask equals running on the kept keys only."""
    rng = np.random.default_rng(11)
    C, T, Hq, Hkv, d = 16, 200, 4, 2, 16
    q, k, v = _rand(rng, C, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
    keep = np.sort(rng.choice(T, 37, replace=False))
    mask = np.full((C, T), DROP)
    mask[:, keep] = 0.0
    got = dense_ref(q, k, v, mask, 0.25)
    want = dense_ref(q, k[keep], v[keep], np.zeros((C, len(keep))), 0.25)
    assert np.max(np.abs(got - want)) < 1e-14


def test_chunked_over_history_equals_one_shot_causal():
    """Chunk after chunk over the accumulated history == one causal pass (SDPA)."""
    rng = np.random.default_rng(3)
    N, Hq, Hkv, d = 300, 4, 2, 16
    q, k, v = _rand(rng, N, Hq, d), _rand(rng, N, Hkv, d), _rand(rng, N, Hkv, d)
    scale = 0.25
    pieces = []
    for s0, C in [(0, 128), (128, 100), (228, 72)]:
        T = s0 + C
        pieces.append(dense_ref(q[s0:T], k[:T], v[:T], causal_mask(s0, C), scale))
    chunked = np.concatenate(pieces)
    qt = torch.from_numpy(q.transpose(1, 0, 2).copy())
    kt = torch.from_numpy(k.transpose(1, 0, 2).copy()).repeat_interleave(2, 0)
    vt = torch.from_numpy(v.transpose(1, 0, 2).copy()).repeat_interleave(2, 0)
    one = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    assert np.max(np.abs(chunked - one.numpy().transpose(1, 0, 2))) < 1e-13


def test_gqa_equals_repeat_kv():
    rng = np.random.default_rng(5)
    C, T, Hq, Hkv, d = 8, 40, 8, 2, 8
    q, k, v = _rand(rng, C, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
    mask = causal_mask(T - C, C).astype(np.float64)
    got = dense_ref(q, k, v, mask, 0.3)
    rep_k = np.repeat(k, Hq // Hkv, axis=1)   # head h reads KV head h // (Hq/Hkv)
    rep_v = np.repeat(v, Hq // Hkv, axis=1)
    want = dense_ref(q, rep_k, rep_v, mask, 0.3)
    assert np.max(np.abs(got - want)) < 1e-15
    # and a wrong mapping (h % Hkv) is detectably different
    alt_k = np.tile(k, (1, Hq // Hkv, 1))
    alt_v = np.tile(v, (1, Hq // Hkv, 1))
    assert np.max(np.abs(dense_ref(q, alt_k, alt_v, mask, 0.3) - got)) > 1e-2


# ---------------------------------------------------------------- closed forms
def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(1)
    C, T, d = 6, 20, 8
    q, k, v = _rand(rng, C, 1, d), _rand(rng, T, 1, d), _rand(rng, T, 1, d)
    mask = np.full((C, T), DROP)
    cols = rng.integers(0, T, C)
    mask[np.arange(C), cols] = rng.normal(0, 5, C)   # any bias: a lone key has weight 1
    o = dense_ref(q, k, v, mask, 0.5)
    assert np.array_equal(o[:, 0, :], v[cols, 0, :])


def test_identical_keys_average_visible_values():
    rng = np.random.default_rng(2)
    C, T, d = 4, 30, 8
    q, v = _rand(rng, C, 1, d), _rand(rng, T, 1, d)
    k = np.repeat(_rand(rng, 1, 1, d), T, axis=0)
    mask = np.where(rng.random((C, T)) < 0.5, DROP, 0.0)
    mask[:, 0] = 0.0
    o = dense_ref(q, k, v, mask, 0.5)
    for i in range(C):
        vis = mask[i] > DROP
        assert np.allclose(o[i, 0], v[vis, 0].mean(axis=0), rtol=0, atol=1e-15)


def test_key_permutation_invariance():
    rng = np.random.default_rng(4)
    C, T, Hq, Hkv, d = 8, 64, 2, 1, 16
    q, k, v = _rand(rng, C, Hq, d), _rand(rng, T, Hkv, d), _rand(rng, T, Hkv, d)
    mask = np.where(rng.random((C, T)) < 0.3, DROP, rng.normal(0, 1, (C, T)))
    perm = rng.permutation(T)
    a = dense_ref(q, k, v, mask, 0.2)
    b = dense_ref(q, k[perm], v[perm], mask[:, perm], 0.2)
    assert np.max(np.abs(a - b)) < 1e-14


# ---------------------------------------------------------------- workload facts
def test_fold_generator_keeps_budget_keys_per_row():
    """2,051 = 512 blocks x 4 keys + 3 recent keys per row past the budget
    ("ANE Prefill Research", What worked, item 2); all causal keys before it."""
    w = make_workload("fold2k5")
    spec = w.spec
    assert spec.fold_budget == 2051
    for idx in range(len(spec.chunks)):
        q_start, C, T, *_rest, mask = w.chunk(idx)
        kept = (mask > DROP).sum(axis=1)
        p = q_start + np.arange(C)
        assert np.all(kept == np.minimum(p + 1, 2051))
        assert not np.any((mask > DROP) & (np.arange(T)[None, :] > p[:, None]))   # never a future key


def test_fold_negative_control_is_not_vacuous():
    """The folded mask must move the oracle output far beyond the GPU tolerance
    relative to a causal-only mask; otherwise the parity check would be vacuous."""
    w = make_workload("fold2k5")
    q_start, C, T, Q, K, V, mask = w.chunk(2)
    q, k, v = (bf16_to_f32(x).astype(np.float64) for x in (Q, K, V))
    rows = np.arange(0, C, 16)
    folded = dense_ref(q, k, v, mask, w.spec.scale, rows=rows)
    causal = dense_ref(q, k, v, causal_mask(q_start, C), w.spec.scale, rows=rows)
    tol = 2e-3 + 1e-2 * np.abs(folded)
    assert np.max(np.abs(folded - causal) / tol) >= 10.0


def test_dense_equiv_pair_counts():
    # config-level accounting: C*P0 + C(C+1)/2 per chunk
    assert sum(dense_equiv_pairs(s, c) for s, c in CONFIGS["tiny"].chunks) == 14368
    assert sum(dense_equiv_pairs(s, c) for s, c in CONFIGS["gqa4k"].chunks) == 9389611
    assert sum(dense_equiv_pairs(s, c) for s, c in CONFIGS["fold2k5"].chunks) == 3126250
    assert sum(dense_equiv_pairs(s, c) for s, c in CONFIGS["sparse32k"].chunks) == 536887296
    assert sum(dense_equiv_pairs(s, c) for s, c in CONFIGS["dense128k"].chunks) == 8590000128


# ---------------------------------------------------------------- folded selection
def _fold_lists(w, q_start, C):
    """Keep lists (blocks of 4 keys) reproducing the fold generator's selection."""
    s = w.spec
    rows = []
    for i in range(C):
        p = q_start + i
        rows.append(list(range(p // s.fold_width + 1)) if p + 1 <= s.fold_budget
                    else [int(c) for c in w.keep_blocks[p]])
    K = max(len(r) for r in rows)
    idx = np.zeros((C, K), dtype=np.int32)
    cnt = np.array([len(r) for r in rows], dtype=np.int32)
    for i, r in enumerate(rows):
        idx[i, :len(r)] = r
    return idx, cnt


def test_fold_mask_equals_generator_mask():
    """Two independent constructions of the folded mask agree bit for bit: the
    generator's per-row column list and the fold of the compacted keep lists."""
    w = make_workload("fold2k5")
    s = w.spec
    for q_start, C in s.chunks:
        idx, cnt = _fold_lists(w, q_start, C)
        got = fold_mask_ref(idx, cnt, q_start, q_start + C, s.fold_width, s.fold_recent)
        assert np.array_equal(got.view(np.uint16), w.mask(q_start, C).view(np.uint16)), q_start


def test_fold_mask_closed_forms():
    # 2 rows at positions 9, 10 over T = 12 keys, blocks of 4, 2 recent keys
    idx = np.array([[0, 2, -1, 7, 0], [1, 2, 9, 9, 9]], dtype=np.int32)
    cnt = np.array([4, 2], dtype=np.int32)     # row 0 reads 4 entries, row 1 two
    m = fold_mask_ref(idx, cnt, 9, 12, 4, 2)
    keep0 = {0, 1, 2, 3, 8, 9}                  # block 0; block 2 clipped at p = 9; -1 and 7 ignored
    keep1 = {4, 5, 6, 7, 8, 9, 10}              # blocks 1 and 2 (clipped at 10); recent 9, 10
    for i, keep in ((0, keep0), (1, keep1)):
        want = np.array([0.0 if t in keep else -30000.0 for t in range(12)], dtype=np.float16)
        assert np.array_equal(m[i], want), i
    # a full-budget row: 512 blocks below the 3 recent keys plus those keys = 2,051 visible
    rng = np.random.default_rng(3)
    p = 5000
    blocks = np.sort(rng.choice((p - 2) // 4, size=512, replace=False)).astype(np.int32)
    m = fold_mask_ref(blocks[None, :], np.array([512], np.int32), p, p + 1, 4, 3)
    assert int((m[0] == 0).sum()) == 2051


# ---------------------------------------------------------------- per-key mask
def test_causal_kmask_composition():
    """Without a per-key mask the composition is the causal mask; dropping keys
    through it equals gathering the others; a finite per-key bias b scales that
    key's weight by e^b (checked against an explicit softmax)."""
    from workloads import causal_mask
    assert np.array_equal(causal_kmask_ref(5, 7, 12).view(np.uint16), causal_mask(5, 7).view(np.uint16))
    rng = np.random.default_rng(12)
    C, T, d, q0 = 6, 14, 8, 8
    q, k, v = rng.standard_normal((C, 1, d)), rng.standard_normal((T, 1, d)), rng.standard_normal((T, 1, d))
    km = np.zeros(T, np.float16)
    km[[2, 5, 11]] = -30000                      # padding keys
    km[7] = np.float16(np.log(3.0))              # a finite bias
    got = dense_ref(q, k, v, causal_kmask_ref(q0, C, T, km), 0.5)
    for i in range(C):
        p = q0 + i
        keep = [t for t in range(p + 1) if t not in (2, 5, 11)]
        s = 0.5 * (k[keep, 0] @ q[i, 0]) + np.array([float(km[t]) for t in keep])
        w = np.exp(s - s.max())
        assert np.allclose(got[i, 0], w @ v[keep, 0] / w.sum(), rtol=1e-13, atol=1e-13)
    # every visible key padded: the row outputs zeros
    km_all = np.full(T, -30000, np.float16)
    assert np.all(dense_ref(q, k, v, causal_kmask_ref(q0, C, T, km_all), 0.5) == 0)


def test_bits_mask_hand_example_and_closed_forms():
    """A hand-packed row: word 0 = 0b1011 keeps keys 0, 1, 3 and drops 2 and 4..31;
    bit 31 of a word is key 31 (sign bit of the int32 word); bit 0 of word 1 is
    key 32.  All bits set equals no mask; no bits set drops every key."""
    T = 40
    bits = np.zeros((3, 2), dtype=np.int32)
    bits[0, 0] = 0b1011
    bits[1, 0] = np.int32(-2 ** 31)             # only bit 31
    bits[1, 1] = 1                              # key 32
    bits[2, :] = -1                             # everything kept (bits past T ignored)
    m = bits_mask_ref(bits, T)
    assert m.shape == (3, T) and m.dtype == np.float16
    assert [t for t in range(T) if m[0, t] == 0] == [0, 1, 3]
    assert [t for t in range(T) if m[1, t] == 0] == [31, 32]
    assert np.all(m[2] == 0)
    assert np.all(m[m != 0] == np.float16(-30000.0))
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((3, 1, 8)), rng.standard_normal((T, 1, 8)), rng.standard_normal((T, 1, 8))
    assert np.array_equal(dense_ref(q, k, v, m, 0.5)[2], dense_ref(q, k, v, np.zeros((3, T), np.float16), 0.5)[2])
    assert np.all(dense_ref(q, k, v, bits_mask_ref(np.zeros((3, 2), np.int32), T), 0.5) == 0)


def test_bits_mask_inverts_the_generator_packing():
    """Two independent constructions: the generator packs a keep pattern with
    numpy's little-endian bit packing, the oracle unpacks bit by bit; the round
    trip gives back the pattern (causal, random, ragged T, padded word rows)."""
    from workloads import pack_keep_bits
    rng = np.random.default_rng(5)
    for C, T, words in ((7, 100, None), (5, 64, 4), (3, 33, None), (2, 1, 3)):
        keep = rng.random((C, T)) < 0.4
        keep[0] = np.arange(T) <= T // 2            # a causal-like row
        bits = pack_keep_bits(keep, words)
        assert bits.dtype == np.int32 and bits.shape == (C, words or -(-T // 32))
        assert np.array_equal(bits_mask_ref(bits, T) == 0, keep)
        if words:                                   # padding words and bits past T are clear
            w = bits.astype(np.int64) & 0xFFFFFFFF
            assert np.all((w[:, -(-T // 32):]) == 0)
    cm = causal_mask(300, 200, 640)
    assert np.array_equal(bits_mask_ref(pack_keep_bits(cm == 0), 640).view(np.uint16), cm.view(np.uint16))
