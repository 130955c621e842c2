"""MI355X-native long-context prefill attention.

Python face of the C ABI (include/prefill_attn.h). Each function takes torch
tensors on the GPU, checks dtypes/shapes/contiguity, and calls the library on
torch's current stream. Outputs are allocated with torch when not supplied.
The calls are asynchronous, like the kernels they enqueue.

    prefill_attn_dense(Q, K, V, mask, scale)                  -> O
    build_pooled_index(K, V, block)                            -> (K_pool, V_pool)
    select_blocks(Q, K_pool, q_start, block, alpha, scale)     -> (sel_idx, sel_cnt)
    prefill_attn_blocksparse(Q, K, V, K_pool, V_pool, sel_idx, sel_cnt, q_start, block, scale) -> O
"""
from __future__ import annotations

import torch

from ._lib import PrefillAttnError, check, lib  # noqa: F401

__all__ = ["prefill_attn_dense", "prefill_attn_dense_workspace", "build_pooled_index",
           "select_blocks", "prefill_attn_blocksparse", "PrefillAttnError", "timing"]


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


def build_pooled_index(K, V, block: int, K_pool=None, V_pool=None):
    """K, V bf16 [T][n_kv][d] -> K_pool, V_pool fp32 [n_kv][ceil(T/block)][d]."""
    _req(K, "K", torch.bfloat16, 3)
    _req(V, "V", torch.bfloat16, 3)
    T, n_kv, d = K.shape
    nb = -(-T // block)
    if K_pool is None:
        K_pool = torch.empty((n_kv, nb, d), dtype=torch.float32, device=K.device)
    if V_pool is None:
        V_pool = torch.empty((n_kv, nb, d), dtype=torch.float32, device=K.device)
    check(lib().build_pooled_index(K.data_ptr(), V.data_ptr(), T, n_kv, d, block,
                                   K_pool.data_ptr(), V_pool.data_ptr(), _stream()),
          "build_pooled_index")
    return K_pool, V_pool


def select_blocks(Q, K_pool, q_start: int, block: int, alpha: float, scale: float,
                  sel_idx=None, sel_cnt=None):
    """-> sel_idx int32 [n_kv][n_qblk][nb], sel_cnt int32 [n_kv][n_qblk]."""
    _req(Q, "Q", torch.bfloat16, 3)
    _req(K_pool, "K_pool", torch.float32, 3)
    C, n_q, d = Q.shape
    n_kv, nb, _ = K_pool.shape
    T = q_start + C
    if nb != -(-T // block):
        raise ValueError(f"K_pool has {nb} blocks; q_start + C = {T} needs {-(-T // block)}")
    n_qblk = (q_start + C - 1) // block - q_start // block + 1
    if sel_idx is None:
        sel_idx = torch.empty((n_kv, n_qblk, nb), dtype=torch.int32, device=Q.device)
    if sel_cnt is None:
        sel_cnt = torch.empty((n_kv, n_qblk), dtype=torch.int32, device=Q.device)
    check(lib().select_blocks(Q.data_ptr(), C, q_start, n_q, n_kv, d, K_pool.data_ptr(), T, block,
                              float(alpha), float(scale), sel_idx.data_ptr(), sel_cnt.data_ptr(),
                              _stream()),
          "select_blocks")
    return sel_idx, sel_cnt


def prefill_attn_blocksparse(Q, K, V, K_pool, V_pool, sel_idx, sel_cnt, q_start: int, block: int,
                             scale: float, O=None):
    """Causal block-sparse attention -> O fp32 [C][n_q][d]."""
    _req(Q, "Q", torch.bfloat16, 3)
    _req(K, "K", torch.bfloat16, 3)
    _req(V, "V", torch.bfloat16, 3)
    _req(K_pool, "K_pool", torch.float32, 3)
    _req(V_pool, "V_pool", torch.float32, 3)
    _req(sel_idx, "sel_idx", torch.int32, 3)
    _req(sel_cnt, "sel_cnt", torch.int32, 2)
    C, n_q, d = Q.shape
    T, n_kv, _ = K.shape
    nb = -(-T // block)
    n_qblk = (q_start + C - 1) // block - q_start // block + 1
    if V.shape != K.shape or K.shape[2] != d:
        raise ValueError("inconsistent Q/K/V shapes")
    if tuple(K_pool.shape) != (n_kv, nb, d) or tuple(V_pool.shape) != (n_kv, nb, d):
        raise ValueError(f"K_pool/V_pool must be {(n_kv, nb, d)}")
    if tuple(sel_idx.shape) != (n_kv, n_qblk, nb) or tuple(sel_cnt.shape) != (n_kv, n_qblk):
        raise ValueError(f"sel_idx/sel_cnt must be {(n_kv, n_qblk, nb)} / {(n_kv, n_qblk)}")
    if O is None:
        O = torch.empty((C, n_q, d), dtype=torch.float32, device=Q.device)
    _req(O, "O", torch.float32, 3)
    check(lib().prefill_attn_blocksparse(Q.data_ptr(), C, q_start, n_q, K.data_ptr(), V.data_ptr(),
                                         T, n_kv, d, K_pool.data_ptr(), V_pool.data_ptr(), block,
                                         sel_idx.data_ptr(), sel_cnt.data_ptr(), float(scale),
                                         O.data_ptr(), _stream()),
          "prefill_attn_blocksparse")
    return O


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
