"""GPU parity: the HIP path, called through the C ABI, against the fp64 CPU oracle.

Bars: pooled index and selection bit-exact; attention elementwise
|gpu - oracle| <= 2e-3 + 1e-2 |oracle|. Inputs are the seeded workloads (or
small seeded cases for edge shapes); no oracle input or expected value comes
from the GPU.
"""
import math
import sys

import numpy as np
import pytest

from oracle import (bits_mask_ref, blocksparse_ref, causal_kmask_ref, dense_ref, fold_mask_ref,
                    pooled_index_ref, select_ref, selection_sets)
from workloads import CONFIGS, bf16_bits, causal_mask, make_workload, pack_keep_bits
from _util import PLANTED32K_ROWS, assert_close, dev_bf16, dev_f16, f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lp():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_prefill_attn_amd as m
    m.lib()
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------- runners
def gpu_dense(lp, q, k, v, mask, scale, ld=None):
    C, T = q.shape[0], k.shape[0]
    if ld is not None and ld != mask.shape[1]:
        padded = np.full((C, ld), np.float16(7.0), dtype=np.float16)   # junk past T must be ignored
        padded[:, :T] = mask[:, :T]
        mask = padded
    O = lp.prefill_attn_dense(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_f16(mask), scale)
    torch.cuda.synchronize()
    return O.cpu().numpy()


def rand_bits(rng, *shape, s=1.0):
    return bf16_bits(rng.standard_normal(shape).astype(np.float32) * s)


# ---------------------------------------------------------------- pooled index
@pytest.mark.parametrize("T,n_kv,d,block", [(4333, 4, 128, 128), (1000, 3, 64, 16), (777, 2, 128, 256),
                                            (64, 1, 64, 64), (1, 2, 128, 128)])
def test_pool_bit_exact(lp, T, n_kv, d, block):
    rng = np.random.default_rng(T + d + block)
    k, v = rand_bits(rng, T, n_kv, d), rand_bits(rng, T, n_kv, d, s=3.0)
    say("pool", T, n_kv, d, block)
    kp, vp = lp.build_pooled_index(dev_bf16(k), dev_bf16(v), block)
    torch.cuda.synchronize()
    rk, rv = pooled_index_ref(f64(k), f64(v), block)
    assert np.array_equal(kp.cpu().numpy().view(np.uint32), rk.view(np.uint32))
    assert np.array_equal(vp.cpu().numpy().view(np.uint32), rv.view(np.uint32))


# ---------------------------------------------------------------- selection
@pytest.mark.parametrize("C,q_start,n_q,n_kv,d,block,alpha", [
    (512, 0, 4, 2, 128, 128, 0.1),
    (300, 37, 4, 1, 128, 64, 0.2),       # chunk starting mid-block
    (256, 256, 8, 2, 64, 32, 0.1),
    (200, 1000, 2, 2, 128, 128, 0.0),    # alpha 0 keeps everything
    (200, 1000, 2, 2, 128, 128, 1.0),    # alpha 1 keeps only the diagonal
    (1, 5000, 4, 4, 128, 16, 0.3),       # a single row over 313 blocks
])
def test_select_bit_exact(lp, C, q_start, n_q, n_kv, d, block, alpha):
    rng = np.random.default_rng(C + q_start)
    T = q_start + C
    q = rand_bits(rng, C, n_q, d, s=2.0)
    k = rand_bits(rng, T, n_kv, d, s=2.0)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("select", C, q_start, n_q, n_kv, d, block, alpha)
    kp, _ = lp.build_pooled_index(dev_bf16(k), dev_bf16(k), block)
    idx, cnt = lp.select_blocks(dev_bf16(q), kp, q_start, block, alpha, scale)
    torch.cuda.synchronize()
    rkp, _ = pooled_index_ref(f64(k), f64(k), block)
    ridx, rcnt = select_ref(f64(q), rkp, q_start, block, alpha, scale)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(idx.cpu().numpy(), ridx)


def _select_pooled(lp, q, kp, q_start, block, alpha, scale, path=None):
    """Selection on a given pooled-key array, GPU vs oracle, bit-exact; `path`:
    the exact path ("listed", "relisted", "pairwise") some voter tile must take."""
    import torch
    Kp = torch.from_numpy(np.ascontiguousarray(kp)).cuda()
    Qd = dev_bf16(q)
    lp.select_path_counts(reset=True)
    idx, cnt = lp.select_blocks(Qd, Kp, q_start, block, alpha, scale)
    paths = lp.select_path_counts(reset=True)
    say("selection paths", paths)
    if path is not None:
        assert paths[path] >= 1, paths
    ridx, rcnt = select_ref(f64(q), kp, q_start, block, alpha, scale)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(idx.cpu().numpy(), ridx)
    return rcnt


@pytest.mark.parametrize("n_q", [1, 16])   # 16 heads: the ambiguous list overflows
def test_select_threshold_edge(lp, n_q):
    """Pooled scores one to ten fp32 ulps either side of M + theta: the filter
    cannot decide them, the fp64 re-evaluation must (strict >)."""
    d, block, q_start, C = 128, 16, 640, 16
    nb = (q_start + C) // block
    scale = float(np.float32(1 / math.sqrt(d)))
    alpha = 0.5
    theta = math.log(alpha) / scale
    q = np.zeros((C, n_q, d), dtype=np.float32)
    q[:, :, 0] = 1.0
    kp = np.zeros((1, nb, d), dtype=np.float32)
    kp[0, 0, 0] = 1.0                                   # the row max M = 1
    edge = np.float32(1.0 + theta)
    vals = []
    for s in range(-10, 10):                            # |s| fp32 ulps away from the edge
        v = edge
        for _ in range(abs(s)):
            v = np.nextafter(v, np.float32(np.inf if s > 0 else -np.inf))
        vals.append(v)
    kp[0, 1:21, 0] = vals
    kp[0, 21:31, 0] = 0.5                               # clearly kept
    kp[0, 31:40, 0] = -100.0                            # clearly dropped
    say("select threshold edge", n_q)
    rcnt = _select_pooled(lp, bf16_bits(q), kp, q_start, block, alpha, scale,
                          path="relisted" if n_q == 16 else "listed")
    assert 10 < rcnt[0, 0] - 1 < 30                     # both sides of the edge occur


@pytest.mark.parametrize("n_q", [2, 8])    # 8 heads: more ambiguous pairs than the list holds
def test_select_identical_pooled_keys(lp, n_q):
    """All pooled keys equal and alpha = 1: every pair ties with the max, so every
    pair is ambiguous and every voter has several near-max candidates."""
    rng = np.random.default_rng(5)
    C, q_start, n_kv, d, block = 200, 1000, 2, 128, 128
    nb = -(-(q_start + C) // block)
    q = rand_bits(rng, C, n_q, d)
    row = rng.standard_normal(d).astype(np.float32)
    kp = np.broadcast_to(row, (n_kv, nb, d)).copy()
    scale = float(np.float32(1 / math.sqrt(d)))
    say("select identical keys", n_q)
    rcnt = _select_pooled(lp, q, kp, q_start, block, 1.0, scale, path="pairwise")
    assert np.all(rcnt == 1)


@pytest.mark.parametrize("d,nc,dense_group", [(128, 1100, False), (128, 1100, True), (64, 700, False)])
def test_select_ambiguous_relisted(lp, d, nc, dense_group):
    """More ambiguous pairs in a voter tile than its list holds, each voter with a
    single near-max candidate: the pairs are formed again a few candidate slices at
    a time and decided exactly against the exact maxima; a group with more pairs
    than the list holds is decided pair by pair. nc candidates span several LDS
    chunks (re-staged) and end in a ragged slice."""
    block, n_q, C = 16, 16, 16
    q_start = nc * block
    scale = float(np.float32(1 / math.sqrt(d)))
    alpha = 0.5
    theta = math.log(alpha) / scale
    q = np.zeros((C, n_q, d), dtype=np.float32)
    q[:, :, 0] = 1.0
    kp = np.zeros((1, nc + 1, d), dtype=np.float32)
    kp[0, :, 0] = np.float32(theta - 12.0)              # clearly dropped
    kp[0, 0, 0] = 1.0                                   # the row max M = 1
    kept = list(range(3, nc, 64))
    kp[0, kept, 0] = 0.5                                # clearly kept
    amb = set(range(7, nc, 32))                         # about four per 128 candidates
    if dense_group:
        amb |= set(range(514, 640, 4))                  # 36 in candidates 512..639
    edge = np.float32(1.0 + theta)
    for i, c in enumerate(sorted(amb)):
        v, s = edge, i % 21 - 10                        # |s| fp32 ulps away from the edge
        for _ in range(abs(s)):
            v = np.nextafter(v, np.float32(np.inf if s > 0 else -np.inf))
        kp[0, c, 0] = v
    say("select ambiguous relisted", d, nc, dense_group)
    rcnt = _select_pooled(lp, bf16_bits(q), kp, q_start, block, alpha, scale, path="relisted")
    base = 2 + len(kept)                                # the max, the clearly kept, the diagonal
    assert base < rcnt[0, 0] < base + len(amb)          # both sides of the edge occur


def test_select_huge_magnitudes(lp):
    """|q| |kbar| beyond the range of the filter's bound: decided in fp64 alone."""
    rng = np.random.default_rng(6)
    C, q_start, n_q, n_kv, d, block = 300, 700, 4, 2, 128, 64
    T = q_start + C
    q = rand_bits(rng, C, n_q, d, s=1e18)
    k = rand_bits(rng, T, n_kv, d, s=1e15)
    kp, _ = pooled_index_ref(f64(k), f64(k), block)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("select huge magnitudes")
    rcnt = _select_pooled(lp, q, kp, q_start, block, 0.1, scale, path="pairwise")
    assert rcnt.min() >= 1


@pytest.mark.parametrize("case", ["subnormal_dims", "past_fp16_range"])
def test_select_fp16_filter_ranges(lp, case):
    """The filter scores in fp16: half of the dims of q and of the keys at 2^-17 of
    the rest (fp16 subnormals, rounded by the conversion and kept by the matrix
    cores), or magnitudes past fp16's largest value (decided in fp64 alone)."""
    rng = np.random.default_rng(8 if case == "subnormal_dims" else 9)
    C, q_start, n_q, n_kv, d, block = 384, 640, 4, 2, 128, 64
    T = q_start + C
    q = rng.standard_normal((C, n_q, d)).astype(np.float32) * 2.0
    k = rng.standard_normal((T, n_kv, d)).astype(np.float32) * 2.0
    if case == "subnormal_dims":
        q[..., d // 2:] *= 2.0 ** -17
        k[..., d // 2:] *= 2.0 ** -17
    else:
        q *= 3e4
    q, k = bf16_bits(q), bf16_bits(k)
    kp, _ = pooled_index_ref(f64(k), f64(k), block)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("select fp16 filter ranges", case)
    rcnt = _select_pooled(lp, q, kp, q_start, block, 0.1, scale)
    assert rcnt.min() >= 1


def test_select_huge_theta(lp):
    """ln(alpha)/scale beyond fp32's comfortable range: decided in fp64 alone."""
    rng = np.random.default_rng(7)
    C, q_start, n_q, n_kv, d, block = 256, 512, 4, 2, 64, 32
    T = q_start + C
    q, k = rand_bits(rng, C, n_q, d), rand_bits(rng, T, n_kv, d)
    kp, _ = pooled_index_ref(f64(k), f64(k), block)
    say("select huge theta")
    _select_pooled(lp, q, kp, q_start, block, 1e-30, 1e-32)


@pytest.mark.parametrize("C,q_start,n_q,n_kv,d,block,alpha,sink,window,tail,s", [
    # voter tiles spread over several workgroups per (KV head, query block) when the
    # pairs are few; the workgroup counts in the comments are those of a 256-CU part
    (512, 3000, 16, 2, 128, 128, 0.1, 0, 0, 0, 2.0),   # 4 per pair; first block's 4th has no voters
    (256, 2048, 8, 1, 64, 64, 0.2, 0, 0, 0, 2.0),      # 2 per pair, head dim 64
    (256, 0, 32, 1, 128, 128, 0.1, 0, 0, 0, 2.0),      # 2 blocks: 2 per pair fills the row exactly
    (512, 1024, 8, 2, 128, 128, 0.1, 256, 2, 1, 2.0),  # kept by rule after the merge
    (300, 700, 8, 2, 128, 128, 0.1, 0, 0, 0, 1e17),    # magnitudes decided in fp64 alone, per tile
    (512, 8192, 16, 2, 128, 256, 0.1, 0, 0, 0, 2.0),   # 8 per pair, two partial words each
])
def test_select_split_voters_bit_exact(lp, C, q_start, n_q, n_kv, d, block, alpha, sink, window, tail, s):
    rng = np.random.default_rng(C + q_start + n_q)
    T = q_start + C
    q = rand_bits(rng, C, n_q, d, s=s)
    k = rand_bits(rng, T, n_kv, d, s=s)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("select split voters", C, q_start, n_q, n_kv, d, block, alpha, sink, window, tail, s)
    kp, _ = lp.build_pooled_index(dev_bf16(k), dev_bf16(k), block)
    idx, cnt = lp.select_blocks(dev_bf16(q), kp, q_start, block, alpha, scale, sink_tokens=sink,
                                window_blocks=window, dense_tail_blocks=tail)
    import torch
    torch.cuda.synchronize()
    rkp, _ = pooled_index_ref(f64(k), f64(k), block)
    ridx, rcnt = select_ref(f64(q), rkp, q_start, block, alpha, scale, sink_tokens=sink,
                            window_blocks=window, dense_tail_blocks=tail)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(idx.cpu().numpy(), ridx)


# ---------------------------------------------------------------- dense: configs
@pytest.mark.parametrize("name", ["tiny", "gqa4k", "fold2k5"])
def test_dense_configs(lp, name):
    w = make_workload(name)
    for idx in range(len(w.spec.chunks)):
        q_start, C, T, q, k, v, mask = w.chunk(idx)
        say("dense", name, "chunk", idx, "C", C, "T", T)
        got = gpu_dense(lp, q, k, v, mask, w.spec.scale)
        want = dense_ref(f64(q), f64(k), f64(v), mask, w.spec.scale)
        assert_close(got, want, f"{name} chunk {idx}")


def test_dense_128k_sampled_rows(lp):
    """Full 128K workload (32 chunks of 4,096, 32/8 heads): chunks 0, 7 and 31 as
    the bench launches them, checked on sampled rows."""
    w = make_workload("dense128k")
    rows = np.concatenate([np.arange(0, 4096, 97), [4095]])
    for idx in (0, 7, 31):
        q_start, C, T, q, k, v, mask = w.chunk(idx)
        say("dense128k chunk", idx, "T", T)
        got = gpu_dense(lp, q, k, v, mask, w.spec.scale)
        want = dense_ref(f64(q[rows]), f64(k), f64(v), mask[rows], w.spec.scale)
        assert_close(got[rows], want, f"dense128k chunk {idx}")


def test_dense_planted_32k_sampled_rows(lp):
    """The dense half of the default benchmark step: the planted 32K tensors in
    4,096-row chunks under fp16 causal masks, launched as the bench launches them.
    The planted positional and topic components give large, structured scores,
    so the lazy-rescale path (scores recomputed from K in global memory) runs at
    full size. Chunks 0, 3 and 7 on sampled rows of every head."""
    w = make_workload("sparse32k")
    s = w.spec
    rows = np.concatenate([np.arange(0, 4096, 127), [4095]])
    for ci in (0, 3, 7):
        q0, C = 4096 * ci, 4096
        T = q0 + C
        mask = causal_mask(q0, C)
        say("planted 32K dense chunk", ci, "T", T)
        got = gpu_dense(lp, w.Q[q0:T], w.K[:T], w.V[:T], mask, s.scale)
        want = dense_ref(f64(w.Q[q0:T][rows]), f64(w.K[:T]), f64(w.V[:T]), mask[rows], s.scale)
        assert_close(got[rows], want, f"planted 32K dense chunk {ci}")


def test_dense_planted_32k_oneshot_sampled_rows(lp):
    """The one-shot dense comparator of the benchmark: one call over the whole
    planted 32K prompt (C = T = 32,768) under its causal mask, sampled rows of
    every head across the prompt."""
    w = make_workload("sparse32k")
    s = w.spec
    N = s.N
    mask = causal_mask(0, N)
    say("planted 32K dense one-shot")
    got = gpu_dense(lp, w.Q, w.K, w.V, mask, s.scale)
    rows = np.concatenate([np.arange(0, N, 1021), [N - 1]])
    want = dense_ref(f64(w.Q[rows]), f64(w.K), f64(w.V), mask[rows], s.scale)
    assert_close(got[rows], want, "planted 32K dense one-shot")


# ---------------------------------------------------------------- dense: edge cases
def _edge(seed, C, T, n_q, n_kv, d, kind):
    rng = np.random.default_rng(seed)
    q = rand_bits(rng, C, n_q, d)
    k = rand_bits(rng, T, n_kv, d)
    v = rand_bits(rng, T, n_kv, d)
    P0 = T - C
    if kind == "causal":
        mask = causal_mask(P0, C, T)
    elif kind == "random":
        m = rng.normal(0.0, 1.0, (C, T))
        m[rng.random((C, T)) < 0.3] = -30000.0
        m[rng.random((C, T)) < 0.05] = -np.inf
        m[rng.random((C, T)) < 0.05] = -1.0e4          # finite, follows the formula
        m[0, :] = -30000.0                               # an all-dropped row -> zeros
        mask = m.astype(np.float16)
    elif kind == "band":
        # keys in [T/4, T/2) are dropped for every row: whole tiles to skip
        mask = causal_mask(P0, C, T)
        mask[:, T // 4: T // 2] = np.float16(-30000.0)
    else:
        raise ValueError(kind)
    return q, k, v, mask


@pytest.mark.parametrize("C,T,n_q,n_kv,d,kind,ld", [
    (1, 1, 1, 1, 128, "causal", None),
    (1, 301, 4, 2, 128, "causal", None),
    (200, 5000, 2, 1, 128, "causal", None),     # few workgroups -> split key range + combine
    (129, 700, 8, 8, 64, "random", None),
    (333, 1500, 4, 1, 128, "random", 1513),     # padded, unaligned mask rows
    (256, 4096, 4, 2, 128, "band", 4104),
    (100, 100, 6, 2, 64, "causal", None),
    (37, 4100, 4, 4, 128, "random", None),      # split path with a random mask
    (300, 2000, 8, 1, 128, "random", None),     # eight heads per workgroup: 32 rows, half a flag row
    (200, 3000, 16, 2, 64, "band", None),       # the same with whole dropped tiles
])
def test_dense_edge_cases(lp, C, T, n_q, n_kv, d, kind, ld):
    q, k, v, mask = _edge(C * 7 + T, C, T, n_q, n_kv, d, kind)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("dense edge", C, T, n_q, n_kv, d, kind, ld)
    got = gpu_dense(lp, q, k, v, mask, scale, ld=ld)
    want = dense_ref(f64(q), f64(k), f64(v), mask, scale)
    assert_close(got, want, f"edge {C},{T},{kind}")
    if kind == "random":
        assert np.all(got[0] == 0.0)


@pytest.mark.parametrize("kind", ["spike", "rising", "falling"])
def test_dense_lazy_rescale(lp, kind):
    """The step loop forms a tile's weights against the running max as it stands
    and raises it only when a row's weights for the tile sum past its bound:
    a late tile whose logits overflow exp2 against the old max ("spike"),
    logits that keep growing ("rising", several raises), and a first tile far
    above the rest ("falling", later weights underflow, no raise)."""
    rng = np.random.default_rng({"spike": 1, "rising": 2, "falling": 3}[kind])
    C, T, n_q, n_kv, d = 256, 4096, 4, 1, 128
    u = rng.standard_normal(d).astype(np.float32)
    q = rng.standard_normal((C, n_q, d)).astype(np.float32) + u
    k = rng.standard_normal((T, n_kv, d)).astype(np.float32)
    if kind == "spike":
        # q.k near 10 |u|^2: ~160 above the rest in log2 units, nearly even across
        # the tile so that many keys share the weight (bf16 weights, as in the method)
        k[3000:3064] = 10.0 * u + 0.25 * k[3000:3064]
    elif kind == "rising":
        k += (np.arange(T, dtype=np.float32) / T * 3.0)[:, None, None] * u
    else:
        k[:64] += 6.0 * u
    v = rng.standard_normal((T, n_kv, d)).astype(np.float32)
    q, k, v = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    mask = np.zeros((C, T), dtype=np.float16)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("dense lazy rescale", kind)
    got = gpu_dense(lp, q, k, v, mask, scale)
    want = dense_ref(f64(q), f64(k), f64(v), mask, scale)
    assert_close(got, want, f"lazy rescale {kind}")


def test_dense_is_deterministic(lp):
    w = make_workload("gqa4k")
    q_start, C, T, q, k, v, mask = w.chunk(1)
    say("determinism gqa4k tail")
    a = gpu_dense(lp, q, k, v, mask, w.spec.scale)
    b = gpu_dense(lp, q, k, v, mask, w.spec.scale)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---------------------------------------------------------------- block-sparse
def _blocksparse_gpu(lp, q, k, v, q_start, block, alpha, scale):
    Qd, Kd, Vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    kp, vp = lp.build_pooled_index(Kd, Vd, block)
    idx, cnt = lp.select_blocks(Qd, kp, q_start, block, alpha, scale)
    O = lp.prefill_attn_blocksparse(Qd, Kd, Vd, kp, vp, idx, cnt, q_start, block, scale)
    torch.cuda.synchronize()
    return kp.cpu().numpy(), vp.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), O.cpu().numpy()


@pytest.mark.parametrize("seed,N,q_start,n_q,n_kv,d,alpha,s", [
    (0, 1024, 0, 4, 2, 128, 0.1, 1.0),
    (1, 1000, 300, 4, 1, 128, 0.2, 1.0),     # chunk starts mid-block, ragged end
    (2, 700, 0, 2, 2, 64, 0.05, 1.0),
    (3, 2048, 1024, 8, 2, 128, 0.5, 0.5),    # small |q|: pooled rows carry real weight
    (4, 1500, 200, 6, 2, 128, 0.1, 1.0),     # three query heads per KV head: one head per workgroup
    (5, 1300, 0, 8, 1, 64, 0.1, 1.0),        # eight query heads per KV head: four workgroups per block
])
def test_blocksparse_small(lp, seed, N, q_start, n_q, n_kv, d, alpha, s):
    rng = np.random.default_rng(seed)
    q = rand_bits(rng, N - q_start, n_q, d, s=s)
    k = rand_bits(rng, N, n_kv, d, s=s)
    v = rand_bits(rng, N, n_kv, d)
    B = 128
    scale = float(np.float32(1 / math.sqrt(d)))
    say("blocksparse small", seed, N, q_start, n_q, n_kv, d, alpha)
    kp, vp, idx, cnt, got = _blocksparse_gpu(lp, q, k, v, q_start, B, alpha, scale)
    rkp, rvp = pooled_index_ref(f64(k), f64(v), B)
    assert np.array_equal(kp.view(np.uint32), rkp.view(np.uint32))
    assert np.array_equal(vp.view(np.uint32), rvp.view(np.uint32))
    ridx, rcnt = select_ref(f64(q), rkp, q_start, B, alpha, scale)
    assert np.array_equal(cnt, rcnt) and np.array_equal(idx, ridx)
    want = blocksparse_ref(f64(q), f64(k), f64(v), rkp, rvp, ridx, rcnt, q_start, B, scale)
    assert_close(got, want, f"blocksparse seed {seed}")


def test_blocksparse_alpha_zero_equals_dense(lp):
    rng = np.random.default_rng(9)
    N, n_q, n_kv, d = 1536, 4, 2, 128
    q, k, v = rand_bits(rng, N, n_q, d), rand_bits(rng, N, n_kv, d), rand_bits(rng, N, n_kv, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("blocksparse alpha 0")
    *_, cnt, got = _blocksparse_gpu(lp, q, k, v, 0, 128, 0.0, scale)
    assert np.all(cnt == np.arange(1, N // 128 + 1)[None, :])
    want = dense_ref(f64(q), f64(k), f64(v), causal_mask(0, N), scale)
    assert_close(got, want, "alpha 0")


def near_threshold_pairs(Q, K_pool, q_start, C, block, alpha, scale, band=1e-4):
    """Voter pairs (row, query head, candidate block) whose exact pooled-score gap
    r - M lies within band * |q| * max|kbar| of ln(alpha)/scale: the selection
    kernel's fp32 filter cannot decide these (its error bound is below that band),
    so each one must have been settled by the exact fp64 re-evaluation."""
    from oracle.blocksparse import threshold
    Hq, d = Q.shape[1], Q.shape[2]
    Hkv = K_pool.shape[0]
    grp = Hq // Hkv
    th = threshold(alpha, scale)
    n = 0
    for g in range(Hkv):
        kb = K_pool[g].astype(np.float64)
        for j in range(q_start // block, (q_start + C - 1) // block + 1):
            if j == 0:
                continue
            r0, r1 = max(j * block, q_start) - q_start, min((j + 1) * block, q_start + C) - q_start
            q = Q[r0:r1, g * grp:(g + 1) * grp].reshape(-1, d)
            r = q @ kb[:j].T
            gap = r - r.max(axis=1, keepdims=True) - th
            e = band * np.linalg.norm(q, axis=1, keepdims=True) * np.linalg.norm(kb[:j], axis=1).max()
            n += int(np.sum(np.abs(gap) <= e))
    return n


@pytest.mark.timeout(900)
def test_blocksparse_32k(lp):
    """Full planted 32K workload as the bench runs it: pooled index and the whole
    selection arrays (every KV head, every query block) bit-exact, and the output
    on the checked rows of every head. Pairs whose gap to the threshold lies
    inside the filter's error band exist at this size, so the exact fp64 path of
    the selection is exercised and compared."""
    w = make_workload("sparse32k")
    s = w.spec
    B = s.block
    say("blocksparse 32K: GPU")
    lp.select_path_counts(reset=True)
    kp, vp, idx, cnt, got = _blocksparse_gpu(lp, w.Q, w.K, w.V, 0, B, s.alpha, s.scale)
    paths = lp.select_path_counts(reset=True)
    say("selection paths", paths)
    # every (KV head, query block) past the first scores its 512 voters as two tiles,
    # and the pairs inside the filter's band are decided in fp64 from the list
    assert paths["tiles"] == s.n_kv * (s.N // B - 1) * 2 and paths["listed"] >= 1, paths
    Q64, K64, V64 = f64(w.Q), f64(w.K), f64(w.V)
    rkp, rvp = pooled_index_ref(K64, V64, B)
    assert np.array_equal(kp.view(np.uint32), rkp.view(np.uint32))
    assert np.array_equal(vp.view(np.uint32), rvp.view(np.uint32))
    say("blocksparse 32K: oracle selection (whole arrays)")
    ridx, rcnt = select_ref(Q64, rkp, 0, B, s.alpha, s.scale)
    assert np.array_equal(cnt, rcnt)
    assert np.array_equal(idx, ridx)
    nb = s.N // B
    say("sparsity", 1.0 - cnt.sum() / (sum(j + 1 for j in range(nb)) * s.n_kv))
    amb = near_threshold_pairs(Q64, rkp, 0, s.N, B, s.alpha, s.scale)
    say("pairs inside the filter band", amb)
    assert amb > 0
    rows = np.array(PLANTED32K_ROWS)
    want = blocksparse_ref(Q64, K64, V64, rkp, rvp, ridx, rcnt, 0, B, s.scale, rows=rows)
    assert_close(got[rows], want, "sparse32k")
    # the same call again: every output bit for bit the same (no atomics decide a value)
    say("blocksparse 32K: second run")
    kp2, vp2, idx2, cnt2, got2 = _blocksparse_gpu(lp, w.Q, w.K, w.V, 0, B, s.alpha, s.scale)
    for a, b in ((kp, kp2), (vp, vp2), (idx, idx2), (cnt, cnt2), (got, got2)):
        assert np.array_equal(np.ascontiguousarray(a).view(np.uint32), np.ascontiguousarray(b).view(np.uint32))


def test_calibrate_alpha_planted_32k(lp):
    """Per-prompt alpha on the planted 32K prompt: the share skipped at the
    returned alpha reaches the target, a slightly smaller alpha falls short, and
    the selection at the returned alpha equals the oracle's on sampled blocks."""
    w = make_workload("sparse32k")
    s = w.spec
    B = s.block
    Qd, Kd, Vd = dev_bf16(w.Q), dev_bf16(w.K), dev_bf16(w.V)
    kp, _ = lp.build_pooled_index(Kd, Vd, B)
    target = 0.80
    a, skip = lp.calibrate_alpha(Qd, kp, 0, B, s.scale, target)
    say("calibrated alpha", a, "skip", skip)
    assert 0.0 < a < s.alpha and skip >= target
    nb = s.N // B
    visible = s.n_kv * nb * (nb + 1) // 2
    _, cnt_below = lp.select_blocks(Qd, kp, 0, B, a * (1 - 1e-6), s.scale)
    assert 1.0 - int(cnt_below.cpu().numpy().astype(np.int64).sum()) / visible < target
    idx, cnt = lp.select_blocks(Qd, kp, 0, B, a, s.scale)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    rkp = pooled_index_ref(f64(w.K), f64(w.V), B)[0]
    a32 = float(np.float32(a))   # the library takes alpha as fp32
    sets = selection_sets(f64(w.Q), rkp, 0, B, a32, s.scale, qblocks=[20, 128, 255])
    for (g, j), kept in sets.items():
        assert cnt[g, j] == len(kept) and np.array_equal(idx[g, j, :len(kept)], kept), (g, j)


# ---------------------------------------------------------------- chunked block-sparse
def test_pool_incremental_bit_exact(lp):
    """Pooling chunk by chunk into one array with spare rows equals pooling the
    whole prefix: the partial block of each earlier chunk is re-pooled, rows past
    the current length are left alone."""
    import torch
    rng = np.random.default_rng(21)
    n_kv, d, block, cap = 2, 128, 128, 12
    k, v = rand_bits(rng, 1400, n_kv, d), rand_bits(rng, 1400, n_kv, d, s=2.0)
    Kd, Vd = dev_bf16(k), dev_bf16(v)
    kp = torch.full((n_kv, cap, d), float("nan"), device="cuda")
    vp = torch.full((n_kv, cap, d), float("nan"), device="cuda")
    say("pool incremental")
    prev = 0
    for T in (300, 1000, 1000, 1400):            # 1000 twice: nothing new to pool
        lp.build_pooled_index(Kd[:T], Vd[:T], block, K_pool=kp, V_pool=vp, b_first=prev // block)
        prev = T
    torch.cuda.synchronize()
    rk, rv = pooled_index_ref(f64(k), f64(v), block)   # 11 blocks of the full 1400 keys
    got_k, got_v = kp.cpu().numpy(), vp.cpu().numpy()
    assert np.array_equal(got_k[:, :11].view(np.uint32), rk.view(np.uint32))
    assert np.array_equal(got_v[:, :11].view(np.uint32), rv.view(np.uint32))
    assert np.isnan(got_k[:, 11:]).all() and np.isnan(got_v[:, 11:]).all()


def _chunked_sparse_gpu(lp, q, k, v, chunks, block, alpha, scale, cap):
    """Chunk-by-chunk block-sparse prefill with one incrementally pooled index."""
    import torch
    Qd, Kd, Vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    n_kv, d = k.shape[1], k.shape[2]
    kp = torch.empty((n_kv, cap, d), device="cuda")
    vp = torch.empty_like(kp)
    O = torch.empty((q.shape[0], q.shape[1], d), device="cuda")
    sels = []
    for q0, C in chunks:
        T = q0 + C
        lp.build_pooled_index(Kd[:T], Vd[:T], block, K_pool=kp, V_pool=vp, b_first=q0 // block)
        idx, cnt = lp.select_blocks(Qd[q0:T], kp, q0, block, alpha, scale)
        lp.prefill_attn_blocksparse(Qd[q0:T], Kd[:T], Vd[:T], kp, vp, idx, cnt, q0, block, scale,
                                    O=O[q0:T])
        sels.append((idx, cnt))
    torch.cuda.synchronize()
    return (kp.cpu().numpy(), vp.cpu().numpy(), [(i.cpu().numpy(), c.cpu().numpy()) for i, c in sels],
            O.cpu().numpy())


def test_blocksparse_chunked_unaligned(lp):
    """Chunks of 1,000 rows (not a multiple of the 128-key block) over a growing
    history: per chunk, selection bit-exact and every output row within tolerance."""
    rng = np.random.default_rng(22)
    N, n_q, n_kv, d, B = 3000, 4, 2, 128, 128
    q, k, v = rand_bits(rng, N, n_q, d), rand_bits(rng, N, n_kv, d), rand_bits(rng, N, n_kv, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    chunks = ((0, 1000), (1000, 1000), (2000, 1000))
    say("blocksparse chunked unaligned")
    kp, vp, sels, got = _chunked_sparse_gpu(lp, q, k, v, chunks, B, 0.1, scale, cap=-(-N // B) + 3)
    rkp, rvp = pooled_index_ref(f64(k), f64(v), B)
    nb = rkp.shape[1]
    assert np.array_equal(kp[:, :nb].view(np.uint32), rkp.view(np.uint32))
    for (q0, C), (idx, cnt) in zip(chunks, sels):
        T = q0 + C
        nbT = -(-T // B)
        # the pooled rows a chunk saw: blocks of its own prefix (the partial last block pooled over T keys)
        pk, pv = pooled_index_ref(f64(k[:T]), f64(v[:T]), B)
        ridx, rcnt = select_ref(f64(q[q0:T]), pk, q0, B, 0.1, scale)
        assert np.array_equal(cnt, rcnt) and np.array_equal(idx, ridx), q0
        want = blocksparse_ref(f64(q[q0:T]), f64(k[:T]), f64(v[:T]), pk, pv, ridx, rcnt, q0, B, scale)
        assert_close(got[q0:T], want, f"chunk at {q0}")
        assert pk.shape[1] == nbT


@pytest.mark.timeout(900)
def test_blocksparse_128k_chunked(lp):
    """The planted 128K prompt in 32 chunks of 4,096 over the growing history, as
    the bench runs it: full pooled index bit-exact, the whole selection arrays of
    chunks 0, 15 and 31 bit-exact, outputs on sampled rows of those chunks."""
    say("blocksparse 128K chunked: generating inputs")
    w = make_workload("sparse128k")
    s = w.spec
    B = s.block
    say("blocksparse 128K chunked: GPU")
    nb = s.N // B
    lp.select_path_counts(reset=True)
    kp, vp, sels, got = _chunked_sparse_gpu(lp, w.Q, w.K, w.V, s.chunks, B, s.alpha, s.scale, cap=nb)
    paths = lp.select_path_counts(reset=True)
    say("selection paths", paths)
    # at about 1,000 candidates some voter tiles hold more pairs inside the fp16
    # filter's band than the list does: the relisting path runs (chunk 31's arrays
    # are compared whole below)
    assert paths["listed"] >= 1 and paths["relisted"] >= 1, paths
    say("blocksparse 128K chunked: oracle")
    K64, V64 = f64(w.K), f64(w.V)
    rkp, rvp = pooled_index_ref(K64, V64, B)
    assert np.array_equal(kp.view(np.uint32), rkp.view(np.uint32))
    assert np.array_equal(vp.view(np.uint32), rvp.view(np.uint32))
    kept = sum(int(c.sum()) for _, c in sels)
    say("sparsity", 1.0 - kept / (nb * (nb + 1) // 2 * s.n_kv))
    for ci in (0, 15, 31):
        q0, C = s.chunks[ci]
        T = q0 + C
        idx, cnt = sels[ci]
        j0 = q0 // B
        nbT = T // B
        Qc = f64(w.Q[q0:T])
        say("blocksparse 128K chunked: oracle selection of chunk", ci)
        ridx, rcnt = select_ref(Qc, rkp[:, :nbT], q0, B, s.alpha, s.scale)
        assert np.array_equal(cnt, rcnt), ci
        assert np.array_equal(idx, ridx), ci
        qblocks = [j0, j0 + 13, j0 + 31]
        rows = np.array([(j - j0) * B + o for j in qblocks for o in (0, 77, 127)])
        want = blocksparse_ref(Qc, K64[:T], V64[:T], rkp[:, :nbT], rvp[:, :nbT], ridx, rcnt, q0, B,
                               s.scale, rows=rows)
        assert_close(got[q0 + rows], want, f"sparse128k chunk {ci}")


# ---------------------------------------------------------------- kept-by-rule selection
@pytest.mark.parametrize("C,q_start,block,alpha,sink,window,tail", [
    (512, 0, 128, 0.1, 256, 2, 0),         # the page's 256-token sinks
    (300, 700, 64, 0.2, 100, 5, 2),        # a partial sink block, a dense tail of two query blocks
    (256, 1024, 32, 1.0, 0, 3, 0),         # alpha 1: window and diagonal only
    (200, 1000, 128, 0.05, 5000, 0, 1),    # sinks past the diagonal are clipped to it
])
def test_select_kept_by_rule_bit_exact(lp, C, q_start, block, alpha, sink, window, tail):
    rng = np.random.default_rng(C + sink)
    T = q_start + C
    n_q, n_kv, d = 4, 2, 128
    q, k = rand_bits(rng, C, n_q, d, s=2.0), rand_bits(rng, T, n_kv, d, s=2.0)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("select rules", C, q_start, block, alpha, sink, window, tail)
    kp, _ = lp.build_pooled_index(dev_bf16(k), dev_bf16(k), block)
    idx, cnt = lp.select_blocks(dev_bf16(q), kp, q_start, block, alpha, scale, sink_tokens=sink,
                                window_blocks=window, dense_tail_blocks=tail)
    import torch
    torch.cuda.synchronize()
    rkp, _ = pooled_index_ref(f64(k), f64(k), block)
    ridx, rcnt = select_ref(f64(q), rkp, q_start, block, alpha, scale, sink_tokens=sink,
                            window_blocks=window, dense_tail_blocks=tail)
    assert np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(idx.cpu().numpy(), ridx)


def test_blocksparse_with_kept_by_rule_selection(lp):
    """Attention over a selection that includes sinks, a window and a dense tail."""
    import torch
    rng = np.random.default_rng(31)
    N, q_start, n_q, n_kv, d, B = 2048, 1024, 4, 2, 128, 128
    q = rand_bits(rng, N - q_start, n_q, d)
    k, v = rand_bits(rng, N, n_kv, d), rand_bits(rng, N, n_kv, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    Qd, Kd, Vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    say("blocksparse rules")
    kp, vp = lp.build_pooled_index(Kd, Vd, B)
    idx, cnt = lp.select_blocks(Qd, kp, q_start, B, 0.2, scale, sink_tokens=256, window_blocks=2,
                                dense_tail_blocks=1)
    O = lp.prefill_attn_blocksparse(Qd, Kd, Vd, kp, vp, idx, cnt, q_start, B, scale)
    torch.cuda.synchronize()
    rkp, rvp = pooled_index_ref(f64(k), f64(v), B)
    ridx, rcnt = select_ref(f64(q), rkp, q_start, B, 0.2, scale, sink_tokens=256, window_blocks=2,
                            dense_tail_blocks=1)
    assert np.array_equal(cnt.cpu().numpy(), rcnt) and np.array_equal(idx.cpu().numpy(), ridx)
    want = blocksparse_ref(f64(q), f64(k), f64(v), rkp, rvp, ridx, rcnt, q_start, B, scale)
    assert_close(O.cpu().numpy(), want, "blocksparse rules")


# ---------------------------------------------------------------- folded selection
def _keep_lists(w, q_start, C):
    s = w.spec
    rows = [list(range(p // s.fold_width + 1)) if p + 1 <= s.fold_budget
            else [int(c) for c in w.keep_blocks[p]] for p in range(q_start, q_start + C)]
    idx = np.zeros((C, max(len(r) for r in rows)), dtype=np.int32)
    for i, r in enumerate(rows):
        idx[i, :len(r)] = r
    return idx, np.array([len(r) for r in rows], dtype=np.int32)


@pytest.mark.parametrize("pad", [0, 3])     # pad 3: rows not 16-byte aligned, scalar stores
def test_fold_keep_mask_bit_exact(lp, pad):
    """The folded fp16 mask equals the oracle's bit for bit on the fold2k5 chunks,
    and dense attention over it equals attention over the host-built mask."""
    import torch
    w = make_workload("fold2k5")
    s = w.spec
    for q_start, C in s.chunks:
        T = q_start + C
        idx, cnt = _keep_lists(w, q_start, C)
        say("fold", q_start, C, pad)
        buf = torch.full((C, T + pad), 7.0, dtype=torch.float16, device="cuda")
        m = lp.fold_keep_mask(torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), q_start, T,
                              s.fold_width, s.fold_recent, mask=buf)
        torch.cuda.synchronize()
        want = fold_mask_ref(idx, cnt, q_start, T, s.fold_width, s.fold_recent)
        got = m.cpu().numpy()
        assert np.array_equal(got[:, :T].view(np.uint16), want.view(np.uint16)), q_start
        assert np.all(got[:, T:] == 7.0)                     # columns past T untouched
    # attention over the device-built mask: identical to the host-built one
    q0, C = s.chunks[-1]
    T = q0 + C
    q, k, v = w.Q[q0:T], w.K[:T], w.V[:T]
    a = gpu_dense(lp, q, k, v, w.mask(q0, C), s.scale)
    idx, cnt = _keep_lists(w, q0, C)
    m = lp.fold_keep_mask(torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), q0, T,
                          s.fold_width, s.fold_recent)
    b = lp.prefill_attn_dense(dev_bf16(q), dev_bf16(k), dev_bf16(v), m, s.scale)
    torch.cuda.synchronize()
    assert np.array_equal(a.view(np.uint32), b.cpu().numpy().view(np.uint32))


def test_fold_keep_mask_malformed_lists(lp):
    """Out-of-range and duplicate block ids, counts past the list width or
    negative, blocks reaching past the row's position."""
    import torch
    rng = np.random.default_rng(41)
    C, q_start, T, width, recent, K = 300, 500, 900, 8, 5, 40
    idx = rng.integers(-5, T // width + 10, size=(C, K)).astype(np.int32)
    idx[:, 5] = idx[:, 4]                                    # duplicates
    cnt = rng.integers(-3, K + 20, size=C).astype(np.int32)
    say("fold malformed")
    m = lp.fold_keep_mask(torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), q_start, T,
                          width, recent)
    torch.cuda.synchronize()
    want = fold_mask_ref(idx, cnt, q_start, T, width, recent)
    assert np.array_equal(m.cpu().numpy().view(np.uint16), want.view(np.uint16))


def _bits_of(mask16, words):
    """The keep bits of an fp16 fold mask (0 = kept), packed as prefill_attn_dense_bits reads them."""
    return pack_keep_bits(mask16 == 0, words=words)


def test_fold_keep_bits_bit_exact(lp):
    """The folded keep bits equal the packing of the oracle's fold mask on the
    fold2k5 chunks (words past ceil(T/32) untouched), and attention over them (the
    pipelined keep-bit loop) and over the device-folded fp16 mask are both within
    tolerance of the oracle's attention under the fold mask."""
    import torch
    w = make_workload("fold2k5")
    s = w.spec
    for q_start, C in s.chunks:
        T = q_start + C
        words = (T + 31) // 32
        idx, cnt = _keep_lists(w, q_start, C)
        say("fold bits", q_start, C)
        buf = torch.full((C, words + 4), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
        bits = lp.fold_keep_bits(torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), q_start, T,
                                 s.fold_width, s.fold_recent, bits=buf)
        torch.cuda.synchronize()
        got = bits.cpu().numpy()
        want = _bits_of(fold_mask_ref(idx, cnt, q_start, T, s.fold_width, s.fold_recent), words)
        assert np.array_equal(got[:, :words], want), q_start
        assert np.all(got[:, words:] == 0x5A5A5A5A)             # words past the row's keys untouched
    q0, C = s.chunks[-1]
    T = q0 + C
    idx, cnt = _keep_lists(w, q0, C)
    ti, tc = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    q, k, v = dev_bf16(w.Q[q0:T]), dev_bf16(w.K[:T]), dev_bf16(w.V[:T])
    a = lp.prefill_attn_dense(q, k, v, lp.fold_keep_mask(ti, tc, q0, T, s.fold_width, s.fold_recent), s.scale)
    b = lp.prefill_attn_dense_bits(q, k, v, lp.fold_keep_bits(ti, tc, q0, T, s.fold_width, s.fold_recent),
                                   s.scale)
    torch.cuda.synchronize()
    rows = np.arange(0, C, 7)                                   # every 7th row, all heads
    want = dense_ref(f64(w.Q[q0:T]), f64(w.K[:T]), f64(w.V[:T]),
                     fold_mask_ref(idx, cnt, q0, T, s.fold_width, s.fold_recent), s.scale, rows=rows)
    assert_close(b.cpu().numpy()[rows], want, "fold bits attention")
    assert_close(a.cpu().numpy()[rows], want, "fold fp16-mask attention")


@pytest.mark.parametrize("C,q_start,T,width,recent,K,seed", [
    (300, 500, 900, 8, 5, 40, 41),            # out-of-range, duplicate and negative entries, odd counts
    (3, 299997, 300000, 64, 100, 50, 42),     # rows over two LDS segments of 262,144 keys
    (40, 60, 100, 1, 0, 70, 43),              # width 1, no recent keys
    (17, 1000, 1017, 100, 37, 12, 44),        # blocks wider than a word, a ragged last word
])
def test_fold_keep_bits_lists(lp, C, q_start, T, width, recent, K, seed):
    import torch
    rng = np.random.default_rng(seed)
    idx = rng.integers(-5, T // width + 10, size=(C, K)).astype(np.int32)
    idx[:, 5] = idx[:, 4]                                    # duplicates
    cnt = rng.integers(-3, K + 20, size=C).astype(np.int32)
    say("fold bits lists", C, q_start, T, width, recent, K)
    bits = lp.fold_keep_bits(torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), q_start, T,
                             width, recent)
    torch.cuda.synchronize()
    words = (T + 31) // 32
    want = _bits_of(fold_mask_ref(idx, cnt, q_start, T, width, recent), words)
    assert np.array_equal(bits.cpu().numpy(), want)


# ---------------------------------------------------------------- causal entry, per-key mask
def test_dense_causal_gqa4k(lp):
    """The causal entry (no mask buffer) on both gqa4k chunks."""
    import torch
    w = make_workload("gqa4k")
    s = w.spec
    for ci, (q0, C) in enumerate(s.chunks):
        T = q0 + C
        say("dense causal gqa4k chunk", ci)
        O = lp.prefill_attn_dense_causal(dev_bf16(w.Q[q0:T]), dev_bf16(w.K[:T]), dev_bf16(w.V[:T]), q0,
                                         s.scale)
        torch.cuda.synchronize()
        heads = np.arange(0, s.n_q, 3)
        want = dense_ref(f64(w.Q[q0:T]), f64(w.K[:T]), f64(w.V[:T]), causal_mask(q0, C), s.scale,
                         heads=heads)
        assert_close(O.cpu().numpy()[:, heads], want, f"causal gqa4k chunk {ci}")


@pytest.mark.parametrize("C,q_start,T,n_q,n_kv,d,pad_from", [
    (700, 300, 1000, 4, 2, 128, None),     # padding and biases scattered over the keys
    (512, 1000, 1700, 8, 2, 128, None),    # T beyond the chunk: keys past each row stay dropped
    (16, 5000, 5016, 4, 1, 128, None),     # few rows: split-key path
    (300, 0, 300, 2, 2, 64, 0),            # leading keys padded: early rows see nothing -> zeros
])
def test_dense_causal_kmask(lp, C, q_start, T, n_q, n_kv, d, pad_from):
    import torch
    rng = np.random.default_rng(C + T)
    q, k, v = rand_bits(rng, C, n_q, d), rand_bits(rng, T, n_kv, d), rand_bits(rng, T, n_kv, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    km = np.zeros(T, np.float16)
    if pad_from is None:
        km[rng.random(T) < 0.1] = -30000
        km[rng.random(T) < 0.05] = np.float16(-1e4)
        sel = rng.random(T) < 0.1
        km[sel] = rng.uniform(-3, 2, size=int(sel.sum())).astype(np.float16)
    else:
        km[pad_from:pad_from + 100] = -30000
    say("dense causal kmask", C, q_start, T, n_q, n_kv, d)
    O = lp.prefill_attn_dense_causal(dev_bf16(q), dev_bf16(k), dev_bf16(v), q_start, scale,
                                     kmask=torch.from_numpy(km).cuda())
    torch.cuda.synchronize()
    want = dense_ref(f64(q), f64(k), f64(v), causal_kmask_ref(q_start, C, T, km), scale)
    got = O.cpu().numpy()
    assert_close(got, want, "causal kmask")
    if pad_from is not None:
        assert np.all(got[:100] == 0)


@pytest.mark.timeout(900)
def test_dense_causal_kv_beyond_2gib(lp):
    """K and V of 1.1M tokens x 8 KV heads x d 128 (2.25 GB each): tiles are
    addressed past 2^31 bytes. Four keys past that boundary (token offsets
    t x 2 KiB >= 2^31) carry a +16 per-key bias and most of every row's weight,
    so the outputs depend on reading them right rather than averaging to near
    zero. Sampled rows of two heads against the oracle."""
    import torch
    T, C, n_kv, d = 1_100_000, 64, 8, 128
    q0 = T - C
    hot = slice(1_090_000, 1_090_004)
    rng = np.random.default_rng(77)
    say("beyond 2 GiB: drawing K, V")
    k = rand_bits(rng, T, n_kv, d)
    v = rand_bits(rng, T, n_kv, d)
    q = rand_bits(rng, C, n_kv, d)
    km = np.zeros(T, dtype=np.float16)
    km[hot] = np.float16(16.0)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("beyond 2 GiB: GPU")
    Kd, Vd = dev_bf16(k), dev_bf16(v)
    O = lp.prefill_attn_dense_causal(dev_bf16(q), Kd, Vd, q0, scale, kmask=dev_f16(km))
    torch.cuda.synchronize()
    got = O.cpu().numpy()
    del Kd, Vd
    say("beyond 2 GiB: oracle")
    rows = np.array([0, 31, 63])
    for g in (0, 7):
        kg, vg = f64(k[:, g:g + 1, :]), f64(v[:, g:g + 1, :])
        qg = f64(q[rows][:, g:g + 1, :])
        for r_i, r in enumerate(rows):
            p = q0 + r
            want = dense_ref(qg[r_i:r_i + 1], kg[:p + 1], vg[:p + 1], km[None, :p + 1], scale)
            assert np.abs(want).max() > 0.1             # not a near-zero average
            assert_close(got[r, g:g + 1], want[0], f"row {r} head {g}")


@pytest.mark.timeout(900)
def test_dense_mask_longest_key_range(lp):
    """The longest key range the mask entry accepts, T = 2^22 - 4096 (the tile-flag
    row at its largest), 64 rows at the end of the history. The mask has every
    tile class along the row: a dropped run of a million keys (DROPPED tiles),
    a +16 bias on four keys and -2 on the next 96 (MIXED), zeros elsewhere
    (ZERO) and the causal edge. The four keys carry most of the weight, so the
    outputs are far from zero and a mishandled tile class moves them past the
    tolerance. Sampled rows of both query heads against the oracle."""
    import torch
    T, C, n_q, n_kv, d = (1 << 22) - 4096, 64, 2, 1, 128
    q0 = T - C
    rng = np.random.default_rng(91)
    say("longest key range: drawing inputs", T)
    k = rand_bits(rng, T, n_kv, d)
    v = rand_bits(rng, T, n_kv, d)
    q = rand_bits(rng, C, n_q, d)
    mask = np.zeros((C, T), dtype=np.float16)
    mask[:, 1_000_000:2_000_000] = np.float16(-30000.0)
    mask[:, 3_000_000:3_000_004] = np.float16(16.0)
    mask[:, 3_000_004:3_000_100] = np.float16(-2.0)
    mask[np.arange(T)[None, :] > (q0 + np.arange(C))[:, None]] = np.float16(-30000.0)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("longest key range: GPU")
    got = gpu_dense(lp, q, k, v, mask, scale)
    say("longest key range: oracle")
    rows = np.array([0, 37, 63])
    want = dense_ref(f64(q), f64(k), f64(v), mask, scale, rows=rows)
    assert np.abs(want).max() > 0.1                     # not a near-zero average
    assert_close(got[rows], want, "longest key range")


# ---------------------------------------------------------------- bit-packed masks
def gpu_dense_bits(lp, q, k, v, bits, scale):
    Bd = torch.from_numpy(np.ascontiguousarray(bits)).cuda()
    O = lp.prefill_attn_dense_bits(dev_bf16(q), dev_bf16(k), dev_bf16(v), Bd, scale)
    torch.cuda.synchronize()
    return O.cpu().numpy()


@pytest.mark.parametrize("C,T,n_q,n_kv,d,kind,words", [
    (237, 4333, 16, 4, 128, "causal", None),     # the gqa4k tail chunk's shape
    (129, 700, 8, 8, 64, "random", None),
    (256, 4100, 4, 2, 128, "band", 136),          # padded rows: junk bits past T must be ignored
    (37, 4100, 4, 4, 128, "random", None),        # split key range + combine
    (300, 1000, 4, 1, 128, "sparse", None),       # ~8% kept: most tiles mixed, some dropped
    (64, 64, 2, 2, 128, "dense", None),           # all kept: every tile plain
])
def test_dense_bits(lp, C, T, n_q, n_kv, d, kind, words):
    rng = np.random.default_rng(C + T + d)
    q, k, v = rand_bits(rng, C, n_q, d), rand_bits(rng, T, n_kv, d), rand_bits(rng, T, n_kv, d)
    t = np.arange(T)[None, :]
    p = (T - C + np.arange(C))[:, None]
    if kind == "causal":
        keep = t <= p
    elif kind == "random":
        keep = rng.random((C, T)) < 0.5
        keep[0] = False                           # an all-dropped row outputs zeros
    elif kind == "band":
        keep = (t <= p) & (t > p - 1500)
    elif kind == "sparse":
        # ~80 keys per row; far fewer makes single bf16-rounded weights dominate
        # and can exceed the tolerance (the same with an fp16 mask)
        keep = rng.random((C, T)) < 0.08
        keep[:, 0] = True
        keep[:, 256:384] = False                  # a fully dropped column of tiles
    else:
        keep = np.ones((C, T), bool)
    bits = pack_keep_bits(keep, words)
    if words is not None:                         # set every bit past T
        w = bits.astype(np.int64) & 0xFFFFFFFF
        for c in range(T // 32, words):
            lo = max(T - 32 * c, 0)
            w[:, c] |= (0xFFFFFFFF >> lo) << lo if lo < 32 else 0
        bits = w.astype(np.uint32).view(np.int32)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("dense bits", C, T, n_q, n_kv, d, kind, words)
    got = gpu_dense_bits(lp, q, k, v, bits, scale)
    want = dense_ref(f64(q), f64(k), f64(v), bits_mask_ref(bits, T), scale)
    assert_close(got, want, f"bits {kind}")
    if kind == "random":
        assert np.all(got[0] == 0.0)
    # the same keep pattern as an fp16 mask (per-step masked loop) is within tolerance too
    same = gpu_dense(lp, q, k, v, np.where(keep, np.float16(0), np.float16(-30000)).astype(np.float16), scale)
    assert_close(same, want, f"fp16 {kind}")


@pytest.mark.parametrize("kind", ["late_low", "sparse_long", "split_long"])
def test_dense_bits_pipelined(lp, kind):
    """The pipelined keep-bit loop over long histories: every key of the first half
    dropped and the rest kept at random with scores near -200 in exp2 units (a row
    has no max until its first kept key, whose weights would underflow against a
    zero max); 10% of 16K keys kept (every step MIXED, ragged end); and a few rows
    whose key range is split over workgroups."""
    rng = np.random.default_rng({"late_low": 61, "sparse_long": 62, "split_long": 63}[kind])
    d, n_q, n_kv = 128, 4, 2
    C, T = {"late_low": (96, 8192), "sparse_long": (64, 16383), "split_long": (8, 20000)}[kind]
    scale = float(np.float32(1 / math.sqrt(d)))
    if kind == "late_low":
        q = np.zeros((C, n_q, d), np.float32)
        q[:, :, 0] = -1568.0                                  # s scale log2(e) ~ -200 for k0 ~ 1
        k = np.zeros((T, n_kv, d), np.float32)
        k[:, :, 0] = 1.0 + 0.01 * rng.standard_normal((T, n_kv))
        q, k = bf16_bits(q), bf16_bits(k)
        keep = np.zeros((C, T), bool)
        keep[:, T // 2:] = rng.random((C, T - T // 2)) < 0.3
    else:
        q, k = rand_bits(rng, C, n_q, d), rand_bits(rng, T, n_kv, d)
        keep = rng.random((C, T)) < 0.1
    v = rand_bits(rng, T, n_kv, d)
    bits = pack_keep_bits(keep)
    say("dense bits pipelined", kind, C, T)
    got = gpu_dense_bits(lp, q, k, v, bits, scale)
    want = dense_ref(f64(q), f64(k), f64(v), bits_mask_ref(bits, T), scale)
    assert_close(got, want, f"bits pipelined {kind}")


# ---------------------------------------------------------------- block sizes other than 128
@pytest.mark.parametrize("B,N,q_start,n_q,n_kv,d,alpha", [
    (16, 700, 300, 4, 2, 128, 0.2),      # four blocks per 64-key step, eight query blocks per workgroup
    (32, 1000, 0, 4, 1, 64, 0.3),
    (64, 1536, 512, 8, 2, 128, 0.3),     # two query blocks per workgroup
    (256, 2048, 300, 4, 2, 128, 0.5),    # two workgroups per query block, chunk starts mid-block
    (256, 2600, 0, 6, 2, 128, 0.7),      # three query heads per KV head
    (16, 2100, 2000, 2, 2, 128, 0.5),    # 100 rows over 132 blocks
])
def test_blocksparse_block_sizes(lp, B, N, q_start, n_q, n_kv, d, alpha):
    rng = np.random.default_rng(B + N + q_start)
    # queries share an N(0,1) direction per query block (plus N(0, 1/4) noise) and
    # keys carry an N(0,1) offset per key block: the rows of a query block vote
    # alike, so the union keeps some blocks and skips others
    nbk = -(-N // B)
    u = rng.standard_normal((nbk, 1, d)).astype(np.float32)
    q = bf16_bits((0.5 * rng.standard_normal((N, n_q, d)).astype(np.float32) + np.repeat(u, B, axis=0)[:N])[q_start:])
    off = rng.standard_normal((nbk, n_kv, d)).astype(np.float32)
    k = bf16_bits(rng.standard_normal((N, n_kv, d)).astype(np.float32) + np.repeat(off, B, axis=0)[:N])
    v = rand_bits(rng, N, n_kv, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("blocksparse block size", B, N, q_start, n_q, n_kv, d, alpha)
    kp, vp, idx, cnt, got = _blocksparse_gpu(lp, q, k, v, q_start, B, alpha, scale)
    rkp, rvp = pooled_index_ref(f64(k), f64(v), B)
    assert np.array_equal(kp.view(np.uint32), rkp.view(np.uint32))
    assert np.array_equal(vp.view(np.uint32), rvp.view(np.uint32))
    ridx, rcnt = select_ref(f64(q), rkp, q_start, B, alpha, scale)
    assert np.array_equal(cnt, rcnt) and np.array_equal(idx, ridx)
    visible = q_start // B + 1 + np.arange(rcnt.shape[1])[None, :]
    assert (rcnt > 1).any() and (rcnt < visible).any()   # some blocks kept below the diagonal, some skipped
    want = blocksparse_ref(f64(q), f64(k), f64(v), rkp, rvp, ridx, rcnt, q_start, B, scale)
    assert_close(got, want, f"blocksparse B={B}")


def test_blocksparse_plain_entry_points(lp):
    """build_pooled_index, select_blocks and prefill_attn_blocksparse called
    through the C ABI directly (not the *_ld forms), block 64, against the oracle."""
    import ctypes
    lib = lp.lib()
    rng = np.random.default_rng(55)
    N, q_start, n_q, n_kv, d, B, alpha = 1200, 400, 4, 2, 128, 64, 0.1
    C, T = N - q_start, N
    q, k, v = rand_bits(rng, C, n_q, d), rand_bits(rng, T, n_kv, d), rand_bits(rng, T, n_kv, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    nb = -(-T // B)
    n_qblk = (q_start + C - 1) // B - q_start // B + 1
    Qd, Kd, Vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    kp = torch.empty((n_kv, nb, d), dtype=torch.float32, device="cuda")
    vp = torch.empty_like(kp)
    idx = torch.empty((n_kv, n_qblk, nb), dtype=torch.int32, device="cuda")
    cnt = torch.empty((n_kv, n_qblk), dtype=torch.int32, device="cuda")
    O = torch.empty((C, n_q, d), dtype=torch.float32, device="cuda")
    need = lib.prefill_attn_blocksparse_workspace(T, n_kv, d)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    say("blocksparse plain entry points")
    assert lib.build_pooled_index(Kd.data_ptr(), Vd.data_ptr(), T, n_kv, d, B, kp.data_ptr(), vp.data_ptr(),
                                  st) == 0
    assert lib.select_blocks(Qd.data_ptr(), C, q_start, n_q, n_kv, d, kp.data_ptr(), T, B, alpha, scale,
                             idx.data_ptr(), cnt.data_ptr(), st) == 0
    assert lib.prefill_attn_blocksparse(Qd.data_ptr(), C, q_start, n_q, Kd.data_ptr(), Vd.data_ptr(), T, n_kv, d,
                                        kp.data_ptr(), vp.data_ptr(), B, idx.data_ptr(), cnt.data_ptr(), scale,
                                        O.data_ptr(), ws.data_ptr(), need, st) == 0
    torch.cuda.synchronize()
    rkp, rvp = pooled_index_ref(f64(k), f64(v), B)
    assert np.array_equal(kp.cpu().numpy().view(np.uint32), rkp.view(np.uint32))
    ridx, rcnt = select_ref(f64(q), rkp, q_start, B, alpha, scale)
    assert np.array_equal(cnt.cpu().numpy(), rcnt) and np.array_equal(idx.cpu().numpy(), ridx)
    want = blocksparse_ref(f64(q), f64(k), f64(v), rkp, rvp, ridx, rcnt, q_start, B, scale)
    assert_close(O.cpu().numpy(), want, "plain entry points")


@pytest.mark.parametrize("B", [128, 64])
def test_blocksparse_malformed_lists(lp, B):
    """Selection lists as a caller might corrupt them: ids outside [0, j),
    duplicates, any order, counts below zero or past the row. The entry point
    reads each list as the set of its valid ids plus the diagonal; the result
    equals the oracle on those cleaned lists."""
    rng = np.random.default_rng(B)
    N, q_start, n_q, n_kv, d = 1500, 200, 4, 2, 128
    C = N - q_start
    q, k, v = rand_bits(rng, C, n_q, d), rand_bits(rng, N, n_kv, d), rand_bits(rng, N, n_kv, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    nb = -(-N // B)
    j0 = q_start // B
    n_qblk = (N - 1) // B - j0 + 1
    idx = rng.integers(-3, nb + 4, size=(n_kv, n_qblk, nb)).astype(np.int32)
    idx[:, :, 1] = idx[:, :, 0]                                 # duplicates
    cnt = rng.integers(-2, nb + 3, size=(n_kv, n_qblk)).astype(np.int32)
    clean_idx = np.zeros_like(idx)
    clean_cnt = np.zeros_like(cnt)
    for g in range(n_kv):
        for jj in range(n_qblk):
            j = j0 + jj
            c = min(max(int(cnt[g, jj]), 0), nb)
            kept = sorted({int(b) for b in idx[g, jj, :c] if 0 <= b < j}) + [j]
            clean_idx[g, jj, :len(kept)] = kept
            clean_cnt[g, jj] = len(kept)
    Qd, Kd, Vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    say("blocksparse malformed lists", B)
    kp, vp = lp.build_pooled_index(Kd, Vd, B)
    O = lp.prefill_attn_blocksparse(Qd, Kd, Vd, kp, vp, torch.from_numpy(idx).cuda(),
                                    torch.from_numpy(cnt).cuda(), q_start, B, scale)
    torch.cuda.synchronize()
    rkp, rvp = pooled_index_ref(f64(k), f64(v), B)
    want = blocksparse_ref(f64(q), f64(k), f64(v), rkp, rvp, clean_idx, clean_cnt, q_start, B, scale)
    assert_close(O.cpu().numpy(), want, f"malformed lists B={B}")


def test_chunked_pipeline_is_deterministic(lp):
    """Pool, select and block-sparse attention over 1,000-row chunks, run twice:
    every output bit for bit the same."""
    rng = np.random.default_rng(23)
    N, n_q, n_kv, d, B = 3000, 8, 2, 128, 64
    q, k, v = rand_bits(rng, N, n_q, d), rand_bits(rng, N, n_kv, d), rand_bits(rng, N, n_kv, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    chunks = ((0, 1000), (1000, 1000), (2000, 1000))
    say("chunked pipeline determinism")
    a = _chunked_sparse_gpu(lp, q, k, v, chunks, B, 0.1, scale, cap=-(-N // B))
    b = _chunked_sparse_gpu(lp, q, k, v, chunks, B, 0.1, scale, cap=-(-N // B))
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    for (i1, c1), (i2, c2) in zip(a[2], b[2]):
        assert np.array_equal(i1, i2) and np.array_equal(c1, c2)
    assert np.array_equal(a[3].view(np.uint32), b[3].view(np.uint32))


# ---------------------------------------------------------------- sharp scores, few keys, value range
@pytest.mark.parametrize("q_start,C,T,n_q,n_kv,sq", [
    (0, 1024, 1024, 8, 2, 1.5),       # causal from position 0: rows 0.. see 1.. keys
    (1024, 1024, 2048, 8, 2, 1.5),
    (0, 512, 512, 4, 4, 2.0),
])
def test_dense_sharp_scores(lp, q_start, C, T, n_q, n_kv, sq):
    """Q and K drawn N(0, sq^2): scores sq^2 times sharper than the workloads',
    so a few keys carry most of a row's weight."""
    rng = np.random.default_rng(C + T)
    d = 128
    q, k, v = rand_bits(rng, C, n_q, d, s=sq), rand_bits(rng, T, n_kv, d, s=sq), rand_bits(rng, T, n_kv, d)
    mask = causal_mask(q_start, C, T)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("dense sharp scores", q_start, C, T, sq)
    got = gpu_dense(lp, q, k, v, mask, scale)
    want = dense_ref(f64(q), f64(k), f64(v), mask, scale)
    worst = assert_close(got, want, f"sharp x{sq}")
    say("worst err/bound", worst)


@pytest.mark.parametrize("kept,sq", [(10, 1.0), (10, 1.5), (3, 1.0)])
def test_dense_few_keys(lp, kept, sq):
    """About `kept` keys per row in a random mask over 2,048 keys, and rows with
    exactly 2 to 5 keys: a handful of comparable weights, where their rounding
    matters most."""
    rng = np.random.default_rng(kept * 10 + int(sq * 10))
    C, T, n_q, n_kv, d = 512, 2048, 4, 2, 128
    q, k, v = rand_bits(rng, C, n_q, d, s=sq), rand_bits(rng, T, n_kv, d, s=sq), rand_bits(rng, T, n_kv, d)
    keep = rng.random((C, T)) < kept / T
    keep[:, 5] = True
    for r in range(8):                         # rows with exactly 2..5 keys
        keep[r] = False
        keep[r, rng.choice(T, size=2 + r % 4, replace=False)] = True
    mask = np.where(keep, np.float16(0), np.float16(-30000)).astype(np.float16)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("dense few keys", kept, sq)
    got = gpu_dense(lp, q, k, v, mask, scale)
    want = dense_ref(f64(q), f64(k), f64(v), mask, scale)
    worst = assert_close(got, want, f"{kept} keys x{sq}")
    say("worst err/bound", worst)


def test_blocksparse_sharp_scores(lp):
    rng = np.random.default_rng(61)
    N, n_q, n_kv, d, B = 2048, 8, 2, 128, 128
    q, k, v = rand_bits(rng, N, n_q, d, s=1.5), rand_bits(rng, N, n_kv, d, s=1.5), rand_bits(rng, N, n_kv, d)
    scale = float(np.float32(1 / math.sqrt(d)))
    say("blocksparse sharp scores")
    kp, vp, idx, cnt, got = _blocksparse_gpu(lp, q, k, v, 0, B, 0.1, scale)
    rkp, rvp = pooled_index_ref(f64(k), f64(v), B)
    ridx, rcnt = select_ref(f64(q), rkp, 0, B, 0.1, scale)
    assert np.array_equal(cnt, rcnt) and np.array_equal(idx, ridx)
    want = blocksparse_ref(f64(q), f64(k), f64(v), rkp, rvp, ridx, rcnt, 0, B, scale)
    worst = assert_close(got, want, "blocksparse sharp")
    say("worst err/bound", worst)


@pytest.mark.parametrize("vs", [3.0e5, 1.0e30, 2.0e-6])
def test_value_range_staging(lp, vs):
    """Values far outside fp16's range (the staging factor 2^-k brings them in and
    the output is scaled back) and tiny values, through the dense and the
    block-sparse entry points."""
    rng = np.random.default_rng(71)
    N, q_start, n_q, n_kv, d, B = 1024, 512, 4, 2, 128, 128
    C = N - q_start
    q, k = rand_bits(rng, C, n_q, d), rand_bits(rng, N, n_kv, d)
    v = rand_bits(rng, N, n_kv, d, s=vs)
    scale = float(np.float32(1 / math.sqrt(d)))
    mask = causal_mask(q_start, C, N)
    say("value range", vs)
    got = gpu_dense(lp, q, k, v, mask, scale)
    want = dense_ref(f64(q), f64(k), f64(v), mask, scale)
    assert_close(got / vs, want / vs, f"dense values x{vs:g}")
    kp, vp, idx, cnt, gs = _blocksparse_gpu(lp, q, k, v, q_start, B, 0.1, scale)
    rkp, rvp = pooled_index_ref(f64(k), f64(v), B)
    ridx, rcnt = select_ref(f64(q), rkp, q_start, B, 0.1, scale)
    want = blocksparse_ref(f64(q), f64(k), f64(v), rkp, rvp, ridx, rcnt, q_start, B, scale)
    assert_close(gs / vs, want / vs, f"blocksparse values x{vs:g}")

