"""Block-sparse prefill attention (FlashPrefill-V2 style), fp64 CPU oracle.

Test infrastructure only (see the package docstring).

Source: "Porting FlashPrefill V2 to Apple silicon for faster prefill", Part I.
The method has three pieces, taken here in the page's order:

1. Pooled index (section "Compress keys before the heavy work"): every block of
   B consecutive keys is summarised by the mean of its keys; the values are
   summarised the same way (the figure legend names the correction a *mean*
   correction).
2. Selection (sections "A cheap map of where the attention lives" and "The
   algorithm starts here"): each query row gets one pooled score per key block;
   a block is worth exact work when its pooled score clears a threshold set by
   alpha relative to the row's hottest block, and the local diagonal block is
   always kept.  Alpha is read in softmax-weight space,
   ``exp(scale*(r_b - M)) > alpha``, i.e. ``r_b - M > ln(alpha)/scale``: with
   alpha = 0 nothing is pruned, as the page's alpha-zero measurement states.
   Rows vote per (KV head, query block of B positions); the block's selection
   is the union of its rows' votes over the group's query heads (the figure
   "Where the kept blocks are" shows one selection map per KV head, with query
   tiles choosing key blocks).
3. Attention (section "Compute the peaks, summarize the rest"): selected blocks
   get exact attention (the diagonal block causally); every other visible block
   enters the same softmax through its pooled row.  A skipped block b stands
   for its B keys, so it carries weight ``B * exp(scale * q.kbar_b - m)`` on the
   mean value ``vbar_b``.

Fixed evaluation orders (so that the GPU can reproduce the integer results and
the fp32 pooled index bit for bit):
* pooled sums run over keys in increasing position, in fp64, then one division
  by the block's key count and one rounding to fp32 (round-to-nearest-even);
* a pooled score ``r_ib = q_i . kbar_b`` sums the head dimensions in increasing
  order in fp64 (each product of a bf16 and an fp32 value is exact in fp64).
"""
from __future__ import annotations

import math

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# -----------------------------------------------------------------------------
# 1. pooled index
# -----------------------------------------------------------------------------
def pooled_index_ref(K, V, block: int):
    """Mean-pooled keys and values.

    K, V [T][Hkv][d] -> K_pool, V_pool [Hkv][ceil(T/B)][d] float32.
    The last block may be partial; its mean divides by its own key count.
    """
    T, Hkv, d = K.shape
    nb = -(-T // block)
    outs = []
    for X in (K, V):
        X = _f64(X)
        pooled = np.zeros((Hkv, nb, d), dtype=np.float32)
        for b in range(nb):
            t0, t1 = b * block, min((b + 1) * block, T)
            acc = np.zeros((Hkv, d), dtype=np.float64)
            for t in range(t0, t1):          # increasing key position
                acc = acc + X[t]
            pooled[:, b, :] = (acc / float(t1 - t0)).astype(np.float32)
        outs.append(pooled)
    return outs[0], outs[1]


# -----------------------------------------------------------------------------
# 2. selection
# -----------------------------------------------------------------------------
def threshold(alpha: float, scale: float) -> float:
    """theta = ln(alpha)/scale in fp64; -inf for alpha = 0 (keep everything)."""
    a = float(np.float32(alpha))
    s = float(np.float32(scale))
    if a == 0.0:
        return -math.inf
    return math.log(a) / s


def pooled_scores(q_rows, kbar) -> np.ndarray:
    """r[i][b] = sum_d q[i][d] * kbar[b][d], summed over d in increasing order."""
    q = _f64(q_rows)
    kb = _f64(kbar)
    r = np.zeros((q.shape[0], kb.shape[0]), dtype=np.float64)
    for dd in range(q.shape[1]):
        r = r + q[:, dd, None] * kb[None, :, dd]
    return r


def selection_votes_ref(q_rows, kbar_visible, alpha: float, scale: float) -> np.ndarray:
    """Votes of a set of query rows over their fully visible blocks.

    q_rows [R][d]; kbar_visible [j][d] (blocks 0..j-1 of the row's KV head).
    Returns bool [R][j]: row i votes for b iff r_ib - max_b r_ib > theta.
    """
    j = kbar_visible.shape[0]
    if j == 0:
        return np.zeros((np.asarray(q_rows).shape[0], 0), dtype=bool)
    r = pooled_scores(q_rows, kbar_visible)
    M = r.max(axis=1, keepdims=True)
    return (r - M) > threshold(alpha, scale)


def rule_blocks(j: int, j_last: int, block: int, sink_tokens: int = 0, window_blocks: int = 0,
                dense_tail_blocks: int = 0) -> set:
    """Blocks b < j kept by rule for query block j (figure "Where the kept blocks
    are": the first tokens as attention sinks, a local window next to the
    diagonal, and the last query tiles attending densely).

    sinks:  every b < ceil(sink_tokens / block);
    window: j - window_blocks <= b < j;
    tail:   every b < j when j > j_last - dense_tail_blocks, j_last being the last
            query block of the call's rows.
    """
    if j > j_last - dense_tail_blocks:
        return set(range(j))
    sinks = set(range(min(j, -(-sink_tokens // block))))
    window = set(range(max(0, j - window_blocks), j))
    return sinks | window


def selection_sets(Q, K_pool, q_start: int, block: int, alpha: float, scale: float,
                   qblocks=None, sink_tokens: int = 0, window_blocks: int = 0,
                   dense_tail_blocks: int = 0) -> dict:
    """{(g, j): sorted list of kept block ids} for the query blocks of a chunk.

    Q [C][Hq][d] holds the chunk's rows at absolute positions q_start..q_start+C-1;
    K_pool [Hkv][Nb][d].  ``qblocks`` optionally restricts the absolute query
    blocks evaluated.  Only rows of this chunk vote.  The kept-by-rule blocks of
    ``rule_blocks`` join the voted ones (all rules off by default).
    """
    C, Hq, d = Q.shape
    Hkv = K_pool.shape[0]
    group = Hq // Hkv
    j0 = q_start // block
    j1 = (q_start + C - 1) // block
    blocks = range(j0, j1 + 1) if qblocks is None else qblocks
    out = {}
    for g in range(Hkv):
        for j in blocks:
            r0 = max(j * block, q_start) - q_start
            r1 = min((j + 1) * block, q_start + C) - q_start
            rows = Q[r0:r1, g * group:(g + 1) * group, :].transpose(1, 0, 2).reshape(-1, d)
            votes = selection_votes_ref(rows, K_pool[g, :j, :], alpha, scale)
            kept = {int(b) for b in np.nonzero(votes.any(axis=0))[0]}
            kept |= rule_blocks(j, j1, block, sink_tokens, window_blocks, dense_tail_blocks)
            out[(g, j)] = sorted(kept) + [j]    # the diagonal block is always kept
    return out


def select_ref(Q, K_pool, q_start: int, block: int, alpha: float, scale: float,
               sink_tokens: int = 0, window_blocks: int = 0, dense_tail_blocks: int = 0):
    """Compacted selection arrays, as the library returns them.

    sel_idx [Hkv][n_qblk][Nb] int32: kept block ids ascending (so the diagonal
    comes last), zero past the count; sel_cnt [Hkv][n_qblk] int32, where
    n_qblk = j(q_start + C - 1) - j(q_start) + 1 and Nb = ceil(T / B).
    """
    C = Q.shape[0]
    Hkv = K_pool.shape[0]
    T = q_start + C
    nb = -(-T // block)
    j0 = q_start // block
    n_qblk = (q_start + C - 1) // block - j0 + 1
    sets = selection_sets(Q, K_pool, q_start, block, alpha, scale, sink_tokens=sink_tokens,
                          window_blocks=window_blocks, dense_tail_blocks=dense_tail_blocks)
    sel_idx = np.zeros((Hkv, n_qblk, nb), dtype=np.int32)
    sel_cnt = np.zeros((Hkv, n_qblk), dtype=np.int32)
    for (g, j), kept in sets.items():
        sel_idx[g, j - j0, :len(kept)] = kept
        sel_cnt[g, j - j0] = len(kept)
    return sel_idx, sel_cnt


# -----------------------------------------------------------------------------
# 3. exact-plus-pooled attention
# -----------------------------------------------------------------------------
def blocksparse_ref(Q, K, V, K_pool, V_pool, sel_idx, sel_cnt, q_start: int, block: int,
                    scale: float, rows=None, heads=None) -> np.ndarray:
    """Block-sparse attention for the chunk rows ``rows`` (default all).

    Row i (absolute position p = q_start + i, query block j = p // B) of head h
    (KV head g) sees:
      exact keys  -- every key of each selected block b < j, and the keys
                     t <= p of its own block j;
      pooled rows -- (kbar_b, vbar_b) with multiplicity B for each b < j that
                     is not selected.
    Output = sum of weighted values / sum of weights, with weights exp(s - m)
    for exact keys and B*exp(sbar - m) for pooled rows.  Returns
    [len(rows)][len(heads)][d] float64.
    """
    C, Hq, d = Q.shape
    Hkv = K.shape[1]
    group = Hq // Hkv
    j0 = q_start // block
    rows = np.arange(C) if rows is None else np.asarray(rows)
    heads = np.arange(Hq) if heads is None else np.asarray(heads)
    sc = float(np.float32(scale))
    out = np.zeros((len(rows), len(heads), d), dtype=np.float64)
    # group the requested rows by query block so each block's key set is built once
    for j in np.unique((q_start + rows) // block):
        in_blk = np.nonzero((q_start + rows) // block == j)[0]
        p = q_start + rows[in_blk]
        kmax = int(p.max()) + 1
        for hi, h in enumerate(heads):
            g = h // group
            kept = [int(b) for b in sel_idx[g, j - j0, :sel_cnt[g, j - j0]]]
            kept_set = set(kept)
            exact_keys = [np.arange(b * block, (b + 1) * block) for b in kept if b < j]
            exact_keys.append(np.arange(j * block, kmax))
            t = np.concatenate(exact_keys)
            q = _f64(Q[rows[in_blk], h, :])
            s = sc * (q @ _f64(K[t, g, :]).T)
            s[t[None, :] > p[:, None]] = -np.inf          # causal inside the diagonal block
            pooled = np.array([b for b in range(j) if b not in kept_set], dtype=np.int64)
            sbar = sc * (q @ _f64(K_pool[g, pooled, :]).T) if len(pooled) else np.zeros((len(p), 0))
            m = np.maximum(s.max(axis=1), sbar.max(axis=1, initial=-np.inf))
            w = np.exp(s - m[:, None])
            wbar = float(block) * np.exp(sbar - m[:, None])
            num = w @ _f64(V[t, g, :])
            den = w.sum(axis=1)
            if len(pooled):
                num += wbar @ _f64(V_pool[g, pooled, :])
                den += wbar.sum(axis=1)
            out[in_blk, hi, :] = num / den[:, None]
    return out
