"""Helpers shared by the tests: device upload of the seeded inputs and the parity bar."""
import numpy as np

from workloads import bf16_to_f32

ATOL, RTOL = 2e-3, 1e-2   # |gpu - oracle| <= ATOL + RTOL * |oracle|, elementwise


def f64(bits):
    return bf16_to_f32(bits).astype(np.float64)


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f16(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float16)).cuda()


def assert_close(got, want, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    bound = ATOL + RTOL * np.abs(want)
    worst = float(np.max(err / bound))
    assert worst <= 1.0, (f"{what}: max err/bound {worst:.3f}, max abs err {err.max():.3e}, "
                          f"rel fro {np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300):.3e}")
    return worst


# Rows of the planted 32K prompt that the block-sparse GPU test checks (all
# heads) and on which the negative controls run: three rows of eight spread
# query blocks, plus rows where an oracle-only scan found dropping the pooled
# correction to move the output most (one or more per KV head).
PLANTED32K_QBLOCKS = (0, 1, 17, 20, 64, 127, 200, 255)
PLANTED32K_ROWS = tuple(sorted({j * 128 + o for j in PLANTED32K_QBLOCKS for o in (0, 63, 127)} |
                               {20543, 24383, 24576, 28672, 31071, 31615, 31807, 32543, 32607, 32767}))
