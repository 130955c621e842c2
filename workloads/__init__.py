"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's checks.

This package holds only input generation (random draws, bf16/fp16 encoding, mask
construction for the workloads).  It contains none of the attention arithmetic:
neither the GPU library nor the CPU oracle is imported here.
"""
from .gen import (  # noqa: F401
    CONFIGS, Workload, bf16_bits, bf16_to_f32, make_workload, causal_mask, folded_mask, pack_keep_bits,
    dense_equiv_pairs, chunk_list, kv_cache_bytes, score_matrix_bytes,
)
