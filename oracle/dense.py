"""Dense chunked prefill attention, written out from its definition (fp64, CPU).

Test infrastructure only (see the package docstring).

What is computed (one chunk, one call):

* A chunk of ``C`` query rows attends over ``T`` keys: the token-major K/V
  history plus the chunk's own keys ("ANE Prefill Research", section "How the
  ANE prefill path works": the chunk's rows, the K/V history and an additive
  mask go in, the attention output comes out).
* The score of row i against key t is ``scale * (q_i . k_t) + mask[i][t]``: an
  additive float mask applied before the softmax ("The Four Principles for
  Optimizing Transformers on the ANE", Principle 3, masking paragraph).  One
  mask ``[C][T]`` serves every head; that page's ``qk_mask`` has no head axis.
* A mask entry at or below -30000 marks a key as omitted: its softmax weight is
  exactly zero, just as a key that was never gathered contributes nothing
  ("ANE Prefill Research", "What worked", item 2 on folding the sparse
  indexer's selection into the mask).  Entries above -30000 are ordinary
  additive biases.  A row whose keys are all omitted outputs zeros.
* Softmax over keys, then the weighted sum of values ("Flash attention on ANE:
  fast long-context prefill", section "Flash attention: the core insight",
  which restates FlashAttention; the tiled GPU kernel must agree with this
  untiled definition).
* Grouped-query attention: query head h reads KV head ``h // (Hq // Hkv)``.

Unlike the GPU path, this materialises the masked score matrix (per head, in
slabs of rows), which is exactly what the pages warn a real implementation must
not do ("Flash attention on ANE", section "The problem with naive attention on
ANE").
"""
from __future__ import annotations

import numpy as np

DROP_AT = -30000.0  # an entry <= this omits the key


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention_weights(q_rows, k, mask_rows, scale) -> np.ndarray:
    """Softmax weights of one head: ``q_rows [R][d]``, ``k [T][d]``,
    ``mask_rows [R][T]`` -> ``[R][T]`` float64.

    Omitted keys get weight exactly 0.0; an all-omitted row is all zeros.
    """
    q = _f64(q_rows)
    kk = _f64(k)
    m = _f64(mask_rows)
    s = float(scale) * (q @ kk.T) + m
    dropped = m <= DROP_AT
    s[dropped] = -np.inf
    row_max = s.max(axis=1, keepdims=True)
    live = np.isfinite(row_max[:, 0])
    w = np.zeros_like(s)
    if live.any():
        e = np.exp(s[live] - row_max[live])
        w[live] = e / e.sum(axis=1, keepdims=True)
    return w


def dense_ref(Q, K, V, mask, scale, rows=None, heads=None, slab: int = 256) -> np.ndarray:
    """Oracle for one chunk of dense prefill attention.

    Q     [C][Hq][d]   query rows of the chunk
    K, V  [T][Hkv][d]  token-major history plus the chunk's keys
    mask  [C][T]       additive mask shared by all heads (fp16 values)
    scale float        softmax scale (the fp32 value the library receives)
    rows  optional sequence of chunk rows to evaluate (default: all)
    heads optional sequence of query heads to evaluate (default: all)

    Returns O [len(rows)][len(heads)][d] in float64.
    """
    C, Hq, d = Q.shape
    T, Hkv, _ = K.shape
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    if mask.shape[0] != C or mask.shape[1] < T:
        raise ValueError("mask must be [C][>=T]")
    group = Hq // Hkv
    rows = np.arange(C) if rows is None else np.asarray(rows)
    heads = np.arange(Hq) if heads is None else np.asarray(heads)
    out = np.zeros((len(rows), len(heads), d), dtype=np.float64)
    for hi, h in enumerate(heads):
        g = h // group
        kg = _f64(K[:, g, :])
        vg = _f64(V[:, g, :])
        for s0 in range(0, len(rows), slab):
            r = rows[s0:s0 + slab]
            w = attention_weights(Q[r, h, :], kg, mask[r, :T], scale)
            out[s0:s0 + slab, hi, :] = w @ vg
    return out


def fold_mask_ref(keep_idx, keep_cnt, q_start: int, T: int, width: int, recent: int) -> np.ndarray:
    """The additive fp16 mask [C][T] of an indexer's compacted selection.

    "ANE Prefill Research", What worked, item 2: the kept keys (keepIndices /
    keepCounts) stay visible and every other key is folded in as -30000.  Row i
    (position p = q_start + i) keeps each key of the listed blocks of `width`
    keys and the `recent` keys ending at p, never a key past p.  Listed blocks
    outside [0, ceil(T/width)) are ignored; at most keep_idx.shape[1] entries of
    a row are read.
    """
    keep_idx = np.asarray(keep_idx)
    C, K = keep_idx.shape if keep_idx.ndim == 2 else (len(keep_cnt), 0)
    nblk = -(-T // width)
    m = np.full((C, T), np.float16(DROP_AT), dtype=np.float16)
    for i in range(C):
        p = q_start + i
        for e in range(min(max(int(keep_cnt[i]), 0), K)):
            c = int(keep_idx[i, e])
            if 0 <= c < nblk:
                m[i, c * width:min(c * width + width, p + 1, T)] = 0
        m[i, max(0, p - recent + 1):min(p + 1, T)] = 0
    return m


def causal_kmask_ref(q_start: int, C: int, T: int, kmask=None) -> np.ndarray:
    """fp16 [C][T]: the causal mask of rows at q_start.. composed by addition with
    a per-key mask kmask [T] ("The Four Principles for Optimizing Transformers on
    the ANE", Principle 3: a (query, key) mask and a per-key padding mask, both
    additive).  Reading: a key dropped by either part (<= -30000) stays dropped;
    otherwise the entry is the per-key bias (the causal part is 0 there)."""
    p = np.arange(q_start, q_start + C)[:, None]
    t = np.arange(T)[None, :]
    k = np.zeros(T, dtype=np.float16) if kmask is None else np.asarray(kmask, dtype=np.float16)
    kdrop = k.astype(np.float64) <= DROP_AT
    drop = (t > p) | kdrop[None, :]
    return np.where(drop, np.float16(DROP_AT), k[None, :]).astype(np.float16)


def bits_mask_ref(bits, T: int) -> np.ndarray:
    """fp16 [C][T] additive mask of a keep/drop mask packed one bit per key.

    "ANE Prefill Research", What worked, item 2: a kept key adds 0, a dropped key
    -30000.  Packing (the library's compact form of such a mask): bit t % 32 of
    the 32-bit word t // 32 of a row, set = kept.  Words are read as unsigned;
    bits of keys >= T do not exist for the row.  Written out bit by bit.
    """
    w = np.asarray(bits).astype(np.int64) & 0xFFFFFFFF
    C = w.shape[0]
    m = np.empty((C, T), dtype=np.float16)
    for t in range(T):
        kept = (w[:, t // 32] >> (t % 32)) & 1
        m[:, t] = np.where(kept == 1, np.float16(0.0), np.float16(DROP_AT))
    return m
