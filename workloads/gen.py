"""Seeded synthetic workloads for long-context prefill attention.

Every workload is drawn from ``numpy.random.Generator(PCG64(seed))`` in a fixed
order: Q, then K, then V, then whatever structure the workload has (the folded
selection of the narrow-chunk case, the planted structure of the block-sparse
case).  Tensors are returned as raw bf16 bit patterns (``uint16``) laid out
token-major, ``[tokens][heads][head_dim]``, which is the layout the C library
takes.  Masks are IEEE fp16 arrays ``[chunk_rows][keys]`` with 0 for a visible
key and -30000 for a dropped one.

The shapes stand in for the prompts the pages measure on (a ~4,333-token prompt
in 4,096 + 237 chunks and a ~2,500-token prompt in 1,024 chunks on the
"ANE Prefill Research" page, the Qwen3-4B attention shapes of the "Porting
FlashPrefill V2 to Apple silicon" page); those prompts themselves are not
available and are not reproduced.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DROPPED = -30000.0  # fp16-exact sentinel for an omitted key


# ----------------------------------------------------------------------------
# encodings
# ----------------------------------------------------------------------------
def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 with round-to-nearest-even; return the bits.

    Works through the array in slices so large inputs need no full-size temporaries."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1).view(np.uint32)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 22
    for s0 in range(0, flat.size, step):
        u = flat[s0:s0 + step]
        t = (u >> np.uint32(16)) & np.uint32(1)
        t += np.uint32(0x7FFF)
        t += u
        t >>= np.uint32(16)
        out[s0:s0 + step] = t
    return out.reshape(x.shape)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# workload specifications
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Spec:
    name: str
    seed: int
    n_q: int
    n_kv: int
    d: int
    N: int                       # tokens in the whole prompt
    chunks: tuple                # ((q_start, C), ...) covering [0, N)
    input_dtype: str = "bf16"    # "fp32" draws are rounded to bf16 before use
    mask: str = "causal"         # "causal" | "folded" | "none" (block-sparse)
    block: int = 128
    alpha: float = 0.1
    structure: str = "normal"    # "normal" | "planted"
    # folded-selection parameters (narrow-chunk case)
    fold_blocks: int = 512
    fold_width: int = 4
    fold_recent: int = 3
    # planted-structure parameters (block-sparse case)
    planted: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d) as the fp32 value passed to the library."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def fold_budget(self) -> int:
        return self.fold_blocks * self.fold_width + self.fold_recent


def chunk_list(N: int, C: int) -> tuple:
    return tuple((s, min(C, N - s)) for s in range(0, N, C))


CONFIGS = {
    # 1 head, d 64, a 64-row chunk at position 192 over 192 history keys; fp32 draws
    "tiny": Spec("tiny", 1, 1, 1, 64, 256, ((192, 64),), input_dtype="fp32"),
    # ~4,333-token prompt: chunk 4,096 at 0, then a 237-row tail at 4,096; GQA 16/4
    "gqa4k": Spec("gqa4k", 2, 16, 4, 128, 4333, ((0, 4096), (4096, 237))),
    # ~2,500 tokens in 1,024 chunks, sparse-indexer selection folded into the mask
    "fold2k5": Spec("fold2k5", 3, 16, 8, 128, 2500, chunk_list(2500, 1024), mask="folded"),
    # block-sparse prefill at 32K, Qwen3-4B attention shapes, alpha 0.1, B 128
    "sparse32k": Spec("sparse32k", 4, 32, 8, 128, 32768, ((0, 32768),), mask="none",
                      structure="planted",
                      planted=dict(Aq=10.0, Ak=5.0, L=6000.0, gamma=6.0, shift=3.0,
                                   n_plants=4, min_j=20, min_gap=16)),
    # 128K dense causal prefill in 4,096-token chunks over the accumulated history
    "dense128k": Spec("dense128k", 5, 32, 8, 128, 131072, chunk_list(131072, 4096)),
    # 128K block-sparse prefill in 4,096-token chunks over the accumulated history
    # (incremental pooled index), same planted structure as the 32K case
    "sparse128k": Spec("sparse128k", 6, 32, 8, 128, 131072, chunk_list(131072, 4096), mask="none",
                       structure="planted",
                       planted=dict(Aq=10.0, Ak=5.0, L=6000.0, gamma=6.0, shift=3.0,
                                    n_plants=4, min_j=20, min_gap=16)),
}


# ----------------------------------------------------------------------------
# masks
# ----------------------------------------------------------------------------
def causal_mask(q_start: int, C: int, T: int | None = None) -> np.ndarray:
    """fp16 [C][T] mask: 0 where key t <= q_start + i, else -30000."""
    if T is None:
        T = q_start + C
    p = np.arange(q_start, q_start + C)[:, None]
    t = np.arange(T)[None, :]
    return np.where(t <= p, np.float16(0.0), np.float16(DROPPED)).astype(np.float16)


def pack_keep_bits(keep, words: int | None = None) -> np.ndarray:
    """int32 [C][words] packing of a boolean keep pattern [C][T]: bit t % 32 of
    word t // 32 set where keep[i][t]; bits past T clear (words defaults to the
    minimum ceil(T / 32))."""
    keep = np.asarray(keep, dtype=bool)
    C, T = keep.shape
    if words is None:
        words = -(-T // 32)
    padded = np.zeros((C, words * 32), dtype=bool)
    padded[:, :T] = keep
    packed = np.packbits(padded, axis=1, bitorder="little")          # bytes, bit j of byte = key 8b + j
    return packed.view("<u4").astype(np.uint32).view(np.int32).reshape(C, words)


def folded_mask(q_start: int, C: int, keep_blocks: dict, spec: Spec, T: int | None = None):
    """fp16 [C][T] mask for the folded sparse-indexer selection.

    Row at absolute position p keeps every causal key while p + 1 <= budget;
    otherwise it keeps the ``fold_recent`` most recent keys and the aligned
    ``fold_width``-key blocks listed in ``keep_blocks[p]``.  Everything else is
    -30000.
    """
    if T is None:
        T = q_start + C
    m = np.full((C, T), np.float16(DROPPED), dtype=np.float16)
    W, R, budget = spec.fold_width, spec.fold_recent, spec.fold_budget
    for i in range(C):
        p = q_start + i
        if p + 1 <= budget:
            m[i, : p + 1] = 0
        else:
            m[i, p - R + 1: p + 1] = 0
            cols = (keep_blocks[p][:, None] * W + np.arange(W)[None, :]).ravel()
            m[i, cols] = 0
    return m


def score_matrix_bytes(tokens: int, heads: int, dtype_bytes: int) -> int:
    """Bytes of a materialised N x N score matrix over all heads."""
    return tokens * tokens * heads * dtype_bytes


def kv_cache_bytes(n_layers: int, n_heads: int, head_dim: int, seq_len: int, dtype_bytes: int) -> int:
    """K plus V cache bytes: 2 * layers * heads * head_dim * tokens * dtype bytes."""
    return 2 * n_layers * n_heads * head_dim * seq_len * dtype_bytes


def dense_equiv_pairs(q_start: int, C: int) -> int:
    """Causally visible (row, key) pairs of a chunk: C*P0 + C(C+1)/2."""
    return C * q_start + C * (C + 1) // 2


# ----------------------------------------------------------------------------
# generation
# ----------------------------------------------------------------------------
class Workload:
    """Materialised inputs of one spec (host numpy arrays)."""

    def __init__(self, spec: Spec, N: int | None = None):
        self.spec = spec
        self.N = spec.N if N is None else N
        self.keep_blocks = {}
        rng = np.random.Generator(np.random.PCG64(spec.seed))
        N, Hq, Hkv, d = self.N, spec.n_q, spec.n_kv, spec.d
        q = rng.standard_normal((N, Hq, d), dtype=np.float32)
        k = rng.standard_normal((N, Hkv, d), dtype=np.float32)
        v = rng.standard_normal((N, Hkv, d), dtype=np.float32)
        if spec.structure == "planted":
            self._plant(rng, q, k)
        if spec.mask == "folded":
            self._draw_fold(rng)
        if spec.input_dtype == "fp32":
            self.q32, self.k32, self.v32 = q, k, v
        self.Q = bf16_bits(q)
        self.K = bf16_bits(k)
        self.V = bf16_bits(v)
        del q, k, v

    # planted structure for the block-sparse case -----------------------------
    def _plant(self, rng, q, k):
        s = self.spec
        P = s.planted
        N, Hq, Hkv, d, B = self.N, s.n_q, s.n_kv, s.d, s.block
        half = d // 2
        group = Hq // Hkv
        # random Fourier features of a Laplace kernel: e(p).e(p') ~ A^2 exp(-|p-p'|/L)
        omega = rng.standard_cauchy(half) / P["L"]
        phi = rng.uniform(0.0, 2.0 * math.pi, half)
        pos = np.arange(N, dtype=np.float64)
        E = math.sqrt(2.0 / half) * np.cos(np.outer(pos, omega) + phi[None, :])
        Eq = (P["Aq"] * E).astype(np.float32)
        Ek = (P["Ak"] * E).astype(np.float32)
        del E
        nqb = (N + B - 1) // B
        topic = rng.standard_normal((Hkv, nqb, half))
        topic /= np.linalg.norm(topic, axis=-1, keepdims=True)
        topic = (P["gamma"] * topic).astype(np.float32)
        blk = np.arange(N) // B
        for h in range(Hq):
            g = h // group
            q[:, h, :half] += Eq
            q[:, h, half:] += topic[g, blk]
        for g in range(Hkv):
            k[:, g, :half] += Ek
        for g in range(Hkv):
            for j in range(P["min_j"], nqb):
                picks = rng.choice(j - P["min_gap"], size=P["n_plants"], replace=False)
                rows = slice(j * B, min((j + 1) * B, N))
                u = q[rows, g * group:(g + 1) * group, :].astype(np.float64).mean(axis=(0, 1))
                u /= np.linalg.norm(u)
                shift = (P["shift"] * u).astype(np.float32)
                for b in np.sort(picks):
                    k[b * B:(b + 1) * B, g, :] += shift

    # folded sparse-indexer selection for the narrow-chunk case ---------------
    def _draw_fold(self, rng):
        s = self.spec
        W, R, budget = s.fold_width, s.fold_recent, s.fold_budget
        for p in range(self.N):
            if p + 1 <= budget:
                continue
            n_cand = (p - (R - 1)) // W   # blocks [Wc, Wc+W-1] lying below the recent keys
            self.keep_blocks[p] = np.sort(rng.choice(n_cand, size=s.fold_blocks, replace=False))

    # per-chunk views ---------------------------------------------------------
    def chunk(self, idx: int):
        """(q_start, C, T, Q_chunk, K[:T], V[:T], mask or None) for chunk idx."""
        q_start, C = self.spec.chunks[idx]
        T = q_start + C
        return q_start, C, T, self.Q[q_start:T], self.K[:T], self.V[:T], self.mask(q_start, C)

    def mask(self, q_start: int, C: int, T: int | None = None):
        if self.spec.mask == "causal":
            return causal_mask(q_start, C, T)
        if self.spec.mask == "folded":
            return folded_mask(q_start, C, self.keep_blocks, self.spec, T)
        return None


_CACHE: dict = {}


def make_workload(name: str, N: int | None = None, cache: bool = True) -> Workload:
    key = (name, N)
    if cache and key in _CACHE:
        return _CACHE[key]
    w = Workload(CONFIGS[name], N)
    if cache:
        _CACHE[key] = w
    return w
