"""A CPU model of the attention kernels' weight rounding (not the oracle; no
GPU). It forms weights the way the kernels do -- per 64-key tile against a
running max that starts at the first tile's max and is raised only when a tile's
rounded weights sum past 2^12 -- rounds them to the weight format, accumulates
rounded weights times values and their sum, and divides. Against the fp64
oracle it shows where each weight format meets the parity bar
|err| <= 2e-3 + 1e-2 |ref|: bf16 weights (8 significant bits) break it on
peaked rows (Q and K at 2x the workloads' scale, rows with 3-10 keys),
fp16 weights (11 bits, what the kernels use) stay far inside it."""
import math

import numpy as np
import pytest

from oracle import dense_ref
from workloads import bf16_bits, bf16_to_f32

LOG2E = 1.4426950408889634


def _bf16(x):
    return bf16_to_f32(bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def _f16(x):
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).astype(np.float64)


def kernel_model(q, k, v, keep, scale, rnd):
    """q [R][d], k, v [T][d] (exact bf16 values), keep [R][T] bool."""
    R, T = keep.shape
    x = (q @ k.T) * (np.float32(scale) * np.float32(LOG2E))
    x = np.where(keep, x, -np.inf)
    O = np.zeros((R, v.shape[1]))
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    for t0 in range(0, T, 64):
        xs = x[:, t0:t0 + 64]
        tmax = xs.max(axis=1)
        m = np.where(np.isfinite(m), m, tmax)
        mu = np.where(np.isfinite(m), m, 0.0)
        P = rnd(np.exp2(xs - mu[:, None]))
        redo = ~(P.sum(axis=1) <= 4096.0)
        if redo.any():
            mn = np.maximum(m, tmax)
            a = np.where(np.isfinite(m), np.exp2(m - np.where(np.isfinite(mn), mn, 0.0)), 1.0)
            O[redo] *= a[redo, None]
            l[redo] *= a[redo]
            m = np.where(redo, mn, m)
            mu = np.where(np.isfinite(m), m, 0.0)
            P = np.where(redo[:, None], rnd(np.exp2(xs - mu[:, None])), P)
        P = np.where(np.isfinite(xs), P, 0.0)
        l += P.sum(axis=1)
        O += P @ v[t0:t0 + 64]
    return np.where(l[:, None] > 0, O / np.where(l > 0, l, 1.0)[:, None], 0.0)


def worst_ratio(seed, R, T, sq, keep_of, fmt):
    rng = np.random.default_rng(seed)
    d = 128
    q = _bf16(rng.standard_normal((R, d)) * sq)
    k = _bf16(rng.standard_normal((T, d)) * sq)
    v = _bf16(rng.standard_normal((T, d)))
    keep = keep_of(rng, R, T)
    scale = float(np.float32(1 / math.sqrt(d)))
    mask = np.where(keep, 0.0, -30000.0)
    want = dense_ref(q[:, None, :], k[:, None, :], v[:, None, :], mask, scale)[:, 0]
    got = kernel_model(q, k, v, keep, scale, _bf16 if fmt == "bf16" else _f16)
    return float(np.max(np.abs(got - want) / (2e-3 + 1e-2 * np.abs(want))))


def causal(rng, R, T):
    return np.arange(T)[None, :] <= (T - R + np.arange(R))[:, None]


def few(n):
    def f(rng, R, T):
        keep = rng.random((R, T)) < n / T
        keep[:, 0] = True
        return keep
    return f


@pytest.mark.parametrize("name,seed,R,T,sq,keep", [
    ("causal tail 2x", 1, 512, 2048, 2.0, causal),
    ("10 keys per row", 2, 512, 1000, 1.0, few(10)),
    ("3 keys per row", 3, 512, 1000, 1.0, few(3)),
])
def test_bf16_weights_break_the_bar_fp16_weights_do_not(name, seed, R, T, sq, keep):
    bf = worst_ratio(seed, R, T, sq, keep, "bf16")
    f16 = worst_ratio(seed, R, T, sq, keep, "fp16")
    assert bf > 1.0, (name, bf)
    assert f16 < 0.35, (name, f16)


def test_workload_scale_long_rows_bf16_within_bar():
    # the workloads' own scale on long causal rows: both formats pass
    assert worst_ratio(4, 512, 1024, 1.0, causal, "fp16") < 0.2
    assert worst_ratio(4, 512, 1024, 1.0, causal, "bf16") < 1.0
