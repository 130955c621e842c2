"""ctypes binding of ``libprefill_attn.so`` (the C ABI in include/prefill_attn.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's kernels. If the
library is missing the import fails loudly -- there is no other implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libprefill_attn.so")

PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_EHIP, PA_EWORKSPACE, PA_ESCRATCH = 0, -1, -2, -3, -4, -5

EXPORTS = {
    # name: (restype, argtypes)
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_select_path_counts": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]),
    "prefill_attn_dense": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int,                    # Q, C, n_q
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,   # K, V, T, n_kv
        ctypes.c_int,                                                   # d
        ctypes.c_void_p, ctypes.c_int64,                                # mask, mask_ld
        ctypes.c_float, ctypes.c_void_p,                                # scale, O
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),            # workspace, bytes, stream
    "prefill_attn_dense_workspace": (ctypes.c_size_t, [ctypes.c_int] * 5),
    "prefill_attn_gather": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,      # Q, C, q_start, n_q
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,   # K, V, T, n_kv
        ctypes.c_int,                                                   # d
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,               # keep_idx, keep_ld, keep_cnt
        ctypes.c_int, ctypes.c_int, ctypes.c_float,                     # width, recent, scale
        ctypes.c_void_p, ctypes.c_void_p]),                             # O, stream
    "prefill_attn_dense_noalloc": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int,                    # Q, C, n_q
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,   # K, V, T, n_kv
        ctypes.c_int,                                                   # d
        ctypes.c_void_p, ctypes.c_int64,                                # mask, mask_ld
        ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]),             # scale, O, stream
    "prefill_attn_dense_noalloc_limit": (ctypes.c_size_t, []),
    "prefill_attn_dense_bits": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int,                    # Q, C, n_q
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,   # K, V, T, n_kv
        ctypes.c_int,                                                   # d
        ctypes.c_void_p, ctypes.c_int64,                                # mask_bits, bits_ld (words)
        ctypes.c_float, ctypes.c_void_p,                                # scale, O
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),            # workspace, bytes, stream
    "prefill_attn_dense_causal": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,      # Q, C, q_start, n_q
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,   # K, V, T, n_kv
        ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, # d, kmask, scale, O
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),            # workspace, bytes, stream
    "build_pooled_index": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "select_blocks": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "prefill_attn_blocksparse": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_float, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),            # workspace, bytes, stream
    "prefill_attn_blocksparse_workspace": (ctypes.c_size_t, [ctypes.c_int] * 3),
    "build_pooled_index_ld": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "select_blocks_ld": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_float,
        ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "prefill_attn_blocksparse_ld": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_float, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),            # workspace, bytes, stream
    "fold_keep_mask": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "fold_keep_bits": (ctypes.c_int, [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "pa_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "pa_timing_reset": (ctypes.c_int, []),
    "pa_timing_read": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_int64)]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m long_context_prefill_attn_amd.build` "
                "(there is no fallback implementation)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


class PrefillAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().pa_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")


def check(status: int, where: str) -> None:
    if status != PA_OK:
        raise PrefillAttnError(status, where)
