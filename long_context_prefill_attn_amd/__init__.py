"""MI355X-native long-context prefill attention.

Python face of the C ABI (include/prefill_attn.h). Each function takes torch
tensors on the GPU, checks dtypes/shapes/contiguity, and calls the library on
torch's current stream. Outputs are allocated with torch when not supplied.
The calls are asynchronous, like the kernels they enqueue.

    prefill_attn_dense(Q, K, V, mask, scale)                  -> O
    prefill_attn_dense_causal(Q, K, V, q_start, scale[, kmask]) -> O
    fold_keep_mask(keep_idx, keep_cnt, q_start, T, width, recent) -> fp16 mask
    build_pooled_index(K, V, block[, K_pool, V_pool, b_first]) -> (K_pool, V_pool)
    select_blocks(Q, K_pool, q_start, block, alpha, scale)     -> (sel_idx, sel_cnt)
    prefill_attn_blocksparse(Q, K, V, K_pool, V_pool, sel_idx, sel_cnt, q_start, block, scale) -> O

The pooled arrays may carry spare block rows ([n_kv][cap][d], cap >= ceil(T/block)):
chunked prefill keeps one pooled index for the whole prompt and pools each chunk's
new blocks with b_first (the *_ld entry points of the C ABI).
"""
from __future__ import annotations

import torch

from ._lib import PrefillAttnError, check, lib  # noqa: F401

__all__ = ["prefill_attn_dense", "prefill_attn_dense_bits", "prefill_attn_dense_causal", "prefill_attn_dense_workspace",
           "prefill_attn_blocksparse_workspace", "build_pooled_index",
           "select_blocks", "prefill_attn_blocksparse", "fold_keep_mask", "fold_keep_bits",
           "prefill_attn_gather",
           "PrefillAttnError", "timing",
           "bisect_alpha", "calibrate_alpha"]


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _req(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def prefill_attn_dense_workspace(C: int, T: int, n_q: int, n_kv: int, d: int) -> int:
    return int(lib().prefill_attn_dense_workspace(C, T, n_q, n_kv, d))


def prefill_attn_dense(Q, K, V, mask, scale: float, O=None, workspace=None):
    """Q bf16 [C][n_q][d]; K, V bf16 [T][n_kv][d]; mask fp16 [C][ld>=T] -> O fp32 [C][n_q][d]."""
    _req(Q, "Q", torch.bfloat16, 3)
    _req(K, "K", torch.bfloat16, 3)
    _req(V, "V", torch.bfloat16, 3)
    _req(mask, "mask", torch.float16, 2)
    C, n_q, d = Q.shape
    T, n_kv, _ = K.shape
    if V.shape != K.shape or K.shape[2] != d or mask.shape[0] != C:
        raise ValueError("inconsistent shapes")
    if O is None:
        O = torch.empty((C, n_q, d), dtype=torch.float32, device=Q.device)
    _req(O, "O", torch.float32, 3)
    need = prefill_attn_dense_workspace(C, T, n_q, n_kv, d)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=Q.device)
    check(lib().prefill_attn_dense(Q.data_ptr(), C, n_q, K.data_ptr(), V.data_ptr(), T, n_kv, d,
                                   mask.data_ptr(), mask.stride(0), float(scale), O.data_ptr(),
                                   workspace.data_ptr(), workspace.numel(), _stream()),
          "prefill_attn_dense")
    return O


def prefill_attn_dense_bits(Q, K, V, mask_bits, scale: float, O=None, workspace=None):
    """Dense chunk under a bit-packed keep mask.

    Q bf16 [C][n_q][d]; K, V bf16 [T][n_kv][d]; mask_bits int32 [C][ld >= ceil(T/32)]
    (bit t%32 of word t//32 set = key t kept, clear = dropped) -> O fp32 [C][n_q][d]."""
    _req(Q, "Q", torch.bfloat16, 3)
    _req(K, "K", torch.bfloat16, 3)
    _req(V, "V", torch.bfloat16, 3)
    _req(mask_bits, "mask_bits", torch.int32, 2)
    C, n_q, d = Q.shape
    T, n_kv, _ = K.shape
    if V.shape != K.shape or K.shape[2] != d or mask_bits.shape[0] != C:
        raise ValueError("inconsistent shapes")
    if mask_bits.shape[1] * 32 < T:
        raise ValueError(f"mask_bits needs at least {(T + 31) // 32} words per row")
    if O is None:
        O = torch.empty((C, n_q, d), dtype=torch.float32, device=Q.device)
    _req(O, "O", torch.float32, 3)
    need = prefill_attn_dense_workspace(C, T, n_q, n_kv, d)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=Q.device)
    check(lib().prefill_attn_dense_bits(Q.data_ptr(), C, n_q, K.data_ptr(), V.data_ptr(), T, n_kv, d,
                                        mask_bits.data_ptr(), mask_bits.stride(0), float(scale),
                                        O.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream()),
          "prefill_attn_dense_bits")
    return O


def prefill_attn_dense_causal(Q, K, V, q_start: int, scale: float, kmask=None, O=None, workspace=None):
    """Causal chunk at positions q_start..q_start+C-1 without a mask buffer.

    Q bf16 [C][n_q][d]; K, V bf16 [T][n_kv][d]; kmask optional fp16 [T] (per-key,
    shared by all rows) -> O fp32 [C][n_q][d]."""
    _req(Q, "Q", torch.bfloat16, 3)
    _req(K, "K", torch.bfloat16, 3)
    _req(V, "V", torch.bfloat16, 3)
    C, n_q, d = Q.shape
    T, n_kv, _ = K.shape
    if V.shape != K.shape or K.shape[2] != d:
        raise ValueError("inconsistent shapes")
    if kmask is not None:
        _req(kmask, "kmask", torch.float16, 1)
        if kmask.shape[0] != T:
            raise ValueError(f"kmask must have T = {T} entries")
    if O is None:
        O = torch.empty((C, n_q, d), dtype=torch.float32, device=Q.device)
    _req(O, "O", torch.float32, 3)
    need = prefill_attn_dense_workspace(C, T, n_q, n_kv, d)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=Q.device)
    check(lib().prefill_attn_dense_causal(Q.data_ptr(), C, q_start, n_q, K.data_ptr(), V.data_ptr(), T,
                                          n_kv, d, kmask.data_ptr() if kmask is not None else None,
                                          float(scale), O.data_ptr(), workspace.data_ptr(),
                                          workspace.numel(), _stream()),
          "prefill_attn_dense_causal")
    return O


def fold_keep_mask(keep_idx, keep_cnt, q_start: int, T: int, width: int, recent: int, mask=None):
    """Fold an indexer's compacted selection into an fp16 mask [C][ld >= T].

    keep_idx int32 [C][K] (kept blocks of `width` keys per row), keep_cnt int32 [C]."""
    _req(keep_idx, "keep_idx", torch.int32, 2)
    _req(keep_cnt, "keep_cnt", torch.int32, 1)
    C, K = keep_idx.shape
    if keep_cnt.shape[0] != C:
        raise ValueError("keep_cnt must have one entry per row")
    if mask is None:
        mask = torch.empty((C, T), dtype=torch.float16, device=keep_idx.device)
    _req(mask, "mask", torch.float16, 2)
    if mask.shape[0] != C or mask.shape[1] < T:
        raise ValueError(f"mask must be [{C}][>= {T}]")
    check(lib().fold_keep_mask(keep_idx.data_ptr() if K else None, K, keep_cnt.data_ptr(), C, q_start,
                               T, width, recent, mask.data_ptr(), mask.stride(0), _stream()),
          "fold_keep_mask")
    return mask


def fold_keep_bits(keep_idx, keep_cnt, q_start: int, T: int, width: int, recent: int, bits=None):
    """Fold an indexer's compacted selection into a bit-packed keep mask int32 [C][ld >= ceil(T/32)]
    (bit t % 32 of word t // 32 set for a kept key), as prefill_attn_dense_bits takes it."""
    _req(keep_idx, "keep_idx", torch.int32, 2)
    _req(keep_cnt, "keep_cnt", torch.int32, 1)
    C, K = keep_idx.shape
    if keep_cnt.shape[0] != C:
        raise ValueError("keep_cnt must have one entry per row")
    words = (T + 31) // 32
    if bits is None:
        bits = torch.empty((C, words), dtype=torch.int32, device=keep_idx.device)
    _req(bits, "bits", torch.int32, 2)
    if bits.shape[0] != C or bits.shape[1] < words:
        raise ValueError(f"bits must be [{C}][>= {words}]")
    check(lib().fold_keep_bits(keep_idx.data_ptr() if K else None, K, keep_cnt.data_ptr(), C, q_start,
                               T, width, recent, bits.data_ptr(), bits.stride(0), _stream()),
          "fold_keep_bits")
    return bits


def prefill_attn_gather(Q, K, V, keep_idx, keep_cnt, q_start: int, width: int, recent: int, scale: float,
                        O=None):
    """Attention over an indexer's compacted selection, scoring only the kept keys.

    Q bf16 [C][n_q][d] (row i at position q_start + i); K, V bf16 [T][n_kv][d];
    keep_idx int32 [C][K] (kept blocks of `width` keys per row), keep_cnt int32 [C]
    -> O fp32 [C][n_q][d]; the same result as prefill_attn_dense over
    fold_keep_mask(keep_idx, keep_cnt, q_start, T, width, recent)."""
    _req(Q, "Q", torch.bfloat16, 3)
    _req(K, "K", torch.bfloat16, 3)
    _req(V, "V", torch.bfloat16, 3)
    _req(keep_idx, "keep_idx", torch.int32, 2)
    _req(keep_cnt, "keep_cnt", torch.int32, 1)
    C, n_q, d = Q.shape
    T, n_kv, _ = K.shape
    Kl = keep_idx.shape[1]
    if V.shape != K.shape or K.shape[2] != d or keep_idx.shape[0] != C or keep_cnt.shape[0] != C:
        raise ValueError("inconsistent shapes")
    if O is None:
        O = torch.empty((C, n_q, d), dtype=torch.float32, device=Q.device)
    _req(O, "O", torch.float32, 3)
    check(lib().prefill_attn_gather(Q.data_ptr(), C, q_start, n_q, K.data_ptr(), V.data_ptr(), T, n_kv, d,
                                    keep_idx.data_ptr() if Kl else None, Kl, keep_cnt.data_ptr(), width,
                                    recent, float(scale), O.data_ptr(), _stream()),
          "prefill_attn_gather")
    return O


def _pooled(P, name, n_kv, nb, d, device):
    """A pooled array [n_kv][cap][d] fp32 with cap >= nb; returns (tensor, cap)."""
    if P is None:
        return torch.empty((n_kv, nb, d), dtype=torch.float32, device=device), nb
    _req(P, name, torch.float32, 3)
    if P.shape[0] != n_kv or P.shape[2] != d or P.shape[1] < nb:
        raise ValueError(f"{name} must be [{n_kv}][>= {nb}][{d}], got {tuple(P.shape)}")
    return P, P.shape[1]


def build_pooled_index(K, V, block: int, K_pool=None, V_pool=None, b_first: int = 0):
    """K, V bf16 [T][n_kv][d] -> K_pool, V_pool fp32 [n_kv][cap][d] (cap >= ceil(T/block)).

    Pools blocks b_first .. ceil(T/block)-1; given arrays with spare capacity keep
    their other rows (chunked prefill: b_first = previous T // block)."""
    _req(K, "K", torch.bfloat16, 3)
    _req(V, "V", torch.bfloat16, 3)
    T, n_kv, d = K.shape
    if V.shape != K.shape:
        raise ValueError("K and V shapes differ")
    nb = -(-T // block)
    K_pool, cap = _pooled(K_pool, "K_pool", n_kv, nb, d, K.device)
    V_pool, cap_v = _pooled(V_pool, "V_pool", n_kv, nb, d, K.device)
    if cap_v != cap:
        raise ValueError("K_pool and V_pool capacities differ")
    check(lib().build_pooled_index_ld(K.data_ptr(), V.data_ptr(), T, n_kv, d, block, b_first,
                                      K_pool.data_ptr(), V_pool.data_ptr(), cap, _stream()),
          "build_pooled_index")
    return K_pool, V_pool


def select_blocks(Q, K_pool, q_start: int, block: int, alpha: float, scale: float,
                  sel_idx=None, sel_cnt=None, sink_tokens: int = 0, window_blocks: int = 0,
                  dense_tail_blocks: int = 0):
    """-> sel_idx int32 [n_kv][n_qblk][nb], sel_cnt int32 [n_kv][n_qblk] (nb = ceil(T/block)).

    K_pool may have spare capacity: [n_kv][cap >= nb][d]. The three rule counts
    keep blocks whatever their scores (see select_blocks_ld in the header)."""
    _req(Q, "Q", torch.bfloat16, 3)
    C, n_q, d = Q.shape
    n_kv = K_pool.shape[0]
    T = q_start + C
    nb = -(-T // block)
    K_pool, cap = _pooled(K_pool, "K_pool", n_kv, nb, d, Q.device)
    n_qblk = (q_start + C - 1) // block - q_start // block + 1
    if sel_idx is None:
        sel_idx = torch.empty((n_kv, n_qblk, nb), dtype=torch.int32, device=Q.device)
    if sel_cnt is None:
        sel_cnt = torch.empty((n_kv, n_qblk), dtype=torch.int32, device=Q.device)
    _req(sel_idx, "sel_idx", torch.int32, 3)
    _req(sel_cnt, "sel_cnt", torch.int32, 2)
    if tuple(sel_idx.shape) != (n_kv, n_qblk, nb) or tuple(sel_cnt.shape) != (n_kv, n_qblk):
        raise ValueError(f"sel_idx/sel_cnt must be {(n_kv, n_qblk, nb)} / {(n_kv, n_qblk)}")
    check(lib().select_blocks_ld(Q.data_ptr(), C, q_start, n_q, n_kv, d, K_pool.data_ptr(), cap, T,
                                 block, float(alpha), float(scale), int(sink_tokens),
                                 int(window_blocks), int(dense_tail_blocks), sel_idx.data_ptr(),
                                 sel_cnt.data_ptr(), _stream()),
          "select_blocks")
    return sel_idx, sel_cnt


def prefill_attn_blocksparse_workspace(T: int, n_kv: int, d: int) -> int:
    return int(lib().prefill_attn_blocksparse_workspace(T, n_kv, d))


def prefill_attn_blocksparse(Q, K, V, K_pool, V_pool, sel_idx, sel_cnt, q_start: int, block: int,
                             scale: float, O=None, workspace=None):
    """Causal block-sparse attention -> O fp32 [C][n_q][d]. K_pool/V_pool may have spare capacity."""
    _req(Q, "Q", torch.bfloat16, 3)
    _req(K, "K", torch.bfloat16, 3)
    _req(V, "V", torch.bfloat16, 3)
    _req(sel_idx, "sel_idx", torch.int32, 3)
    _req(sel_cnt, "sel_cnt", torch.int32, 2)
    C, n_q, d = Q.shape
    T, n_kv, _ = K.shape
    nb = -(-T // block)
    n_qblk = (q_start + C - 1) // block - q_start // block + 1
    if V.shape != K.shape or K.shape[2] != d:
        raise ValueError("inconsistent Q/K/V shapes")
    K_pool, cap = _pooled(K_pool, "K_pool", n_kv, nb, d, Q.device)
    V_pool, cap_v = _pooled(V_pool, "V_pool", n_kv, nb, d, Q.device)
    if cap_v != cap:
        raise ValueError("K_pool and V_pool capacities differ")
    if tuple(sel_idx.shape) != (n_kv, n_qblk, nb) or tuple(sel_cnt.shape) != (n_kv, n_qblk):
        raise ValueError(f"sel_idx/sel_cnt must be {(n_kv, n_qblk, nb)} / {(n_kv, n_qblk)}")
    if O is None:
        O = torch.empty((C, n_q, d), dtype=torch.float32, device=Q.device)
    _req(O, "O", torch.float32, 3)
    need = prefill_attn_blocksparse_workspace(T, n_kv, d)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=Q.device)
    check(lib().prefill_attn_blocksparse_ld(Q.data_ptr(), C, q_start, n_q, K.data_ptr(), V.data_ptr(),
                                            T, n_kv, d, K_pool.data_ptr(), V_pool.data_ptr(), cap,
                                            block, sel_idx.data_ptr(), sel_cnt.data_ptr(),
                                            float(scale), O.data_ptr(), workspace.data_ptr(),
                                            workspace.numel(), _stream()),
          "prefill_attn_blocksparse")
    return O


def bisect_alpha(skip_of, target: float, lo: float = 0.0, hi: float = 1.0, iters: int = 30):
    """Smallest alpha in [lo, hi] whose skipped share reaches `target`, by bisection.

    skip_of(alpha) -> skipped share of the visible blocks; it must be
    non-decreasing in alpha. Selection sets shrink as alpha grows (a block kept
    at some alpha is kept at every smaller one), so this holds for selections.
    Returns (alpha, skip_of(alpha)). If even `hi` falls short, returns hi and its share."""
    s_hi = skip_of(hi)
    if s_hi < target:
        return hi, s_hi
    s_lo = skip_of(lo)
    if s_lo >= target:
        return lo, s_lo
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        s = skip_of(mid)
        if s >= target:
            hi, s_hi = mid, s
        else:
            lo = mid
    return hi, s_hi


def calibrate_alpha(Q, K_pool, q_start: int, block: int, scale: float, target_skip: float,
                    iters: int = 30, sink_tokens: int = 0, window_blocks: int = 0,
                    dense_tail_blocks: int = 0):
    """Per-prompt alpha: the smallest alpha whose selection skips at least
    `target_skip` of this call's visible blocks. The FlashPrefill port picks alpha
    per prompt length this way, to match a measured skip share ("Porting
    FlashPrefill V2 to Apple silicon", A cheap map of where the attention lives).
    Each probe is one select_blocks call on the device; only the per-block counts
    (n_kv x n_qblk integers) come back to the host. Returns (alpha, skip)."""
    C = Q.shape[0]
    n_kv = K_pool.shape[0]
    j0, j1 = q_start // block, (q_start + C - 1) // block
    visible = n_kv * sum(j + 1 for j in range(j0, j1 + 1))
    sel_idx = sel_cnt = None

    def skip_of(alpha):
        nonlocal sel_idx, sel_cnt
        sel_idx, sel_cnt = select_blocks(Q, K_pool, q_start, block, alpha, scale, sel_idx, sel_cnt,
                                         sink_tokens, window_blocks, dense_tail_blocks)
        kept = int(sel_cnt.cpu().numpy().astype("int64").sum())
        return 1.0 - kept / visible

    return bisect_alpha(skip_of, target_skip, 0.0, 1.0, iters)


def select_path_counts(reset: bool = False) -> dict:
    """Voter tiles scored by the selection on the current device since the last
    reset, and how many took each exact path (see pa_select_path_counts):
    {"tiles", "listed", "relisted", "pairwise"}. Waits for the device."""
    import ctypes
    out = (ctypes.c_int64 * 4)()
    check(lib().pa_select_path_counts(ctypes.addressof(out), 1 if reset else 0), "pa_select_path_counts")
    return dict(zip(("tiles", "listed", "relisted", "pairwise"), (int(v) for v in out)))


class timing:
    """Per-kernel HIP-event timing inside the library (see pa_timing_* in the header)."""

    @staticmethod
    def enable(on: bool = True) -> None:
        check(lib().pa_timing_enable(1 if on else 0), "pa_timing_enable")

    @staticmethod
    def reset() -> None:
        check(lib().pa_timing_reset(), "pa_timing_reset")

    @staticmethod
    def read(kernel: str):
        import ctypes
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        check(lib().pa_timing_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)), "pa_timing_read")
        return ms.value, n.value
