"""The allocation-free dense entry point (prefill_attn_dense_noalloc), called
through the C ABI, against the workspace entry point prefill_attn_dense on the
same inputs: two calls in a row on one GPU, the second smaller (and taking the
split-key path, so partial results share the static scratch with the first
call's leftovers). Outputs must be bit-identical to the workspace entry's and
within the oracle tolerance."""
import ctypes
import math

import numpy as np
import pytest

from oracle import dense_ref
from workloads import bf16_bits, causal_mask
from _util import assert_close, dev_bf16, dev_f16, f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _case(rng, C, q_start, n_q, n_kv, d):
    T = q_start + C
    q = bf16_bits(rng.standard_normal((C, n_q, d)).astype(np.float32))
    k = bf16_bits(rng.standard_normal((T, n_kv, d)).astype(np.float32))
    v = bf16_bits(rng.standard_normal((T, n_kv, d)).astype(np.float32))
    return q, k, v, causal_mask(q_start, C, T), float(np.float32(1 / math.sqrt(d)))


def test_noalloc_matches_workspace_entry():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_prefill_attn_amd as lp
    lib = lp.lib()
    rng = np.random.default_rng(97)
    for C, q_start, n_q, n_kv, d in ((1024, 2048, 8, 2, 128), (37, 4063, 4, 2, 64)):
        T = q_start + C
        need = lp.prefill_attn_dense_workspace(C, T, n_q, n_kv, d)
        assert 0 < need <= lib.prefill_attn_dense_noalloc_limit()
        q, k, v, mask, scale = _case(rng, C, q_start, n_q, n_kv, d)
        Qd, Kd, Vd, Md = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f16(mask)
        print("noalloc case", C, q_start, n_q, n_kv, d, flush=True)
        ref = lp.prefill_attn_dense(Qd, Kd, Vd, Md, scale)
        O = torch.full((C, n_q, d), float("nan"), dtype=torch.float32, device="cuda")
        st = torch.cuda.current_stream().cuda_stream
        assert lib.prefill_attn_dense_noalloc(Qd.data_ptr(), C, n_q, Kd.data_ptr(), Vd.data_ptr(), T, n_kv, d,
                                              Md.data_ptr(), Md.stride(0), scale, O.data_ptr(), st) == 0
        torch.cuda.synchronize()
        got, want_ws = O.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want_ws.view(np.uint32))
        assert_close(got, dense_ref(f64(q), f64(k), f64(v), mask, scale), f"noalloc C={C}")
