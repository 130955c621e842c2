"""The entry points under HIP graph capture (as `bench.py --graph` times them):
a captured call sequence, replayed several times with eager work and
synchronizations between the replays, writes exactly what the eager calls
wrote (the kernels are deterministic), every replay. No oracle here: the eager
results are checked against the oracle by the parity tests."""
import numpy as np
import pytest

from workloads import chunk_list, make_workload
from _util import dev_bf16

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


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_checks(g, outs, want, eager_between):
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o.view(torch.int32) if o.is_floating_point() else o, w), f"replay {rep}"
        eager_between()           # other work on the device between replays
        torch.cuda.synchronize()


def test_graph_folded_chunks(lp):
    """fold2k5: each chunk's lists folded into keep bits, then dense attention over
    them (split key ranges and the combine on the short chunk), all chunks in one graph."""
    w = make_workload("fold2k5")
    s = w.spec
    Q, K, V = dev_bf16(w.Q), dev_bf16(w.K), dev_bf16(w.V)
    O = torch.empty((w.N, s.n_q, s.d), dtype=torch.float32, device="cuda")
    calls = []
    for q0, C in s.chunks:
        T = q0 + C
        rows = [list(range(p // s.fold_width + 1)) if p + 1 <= s.fold_budget else [int(c) for c in w.keep_blocks[p]]
                for p in range(q0, T)]
        idx = np.zeros((C, max(len(r) for r in rows)), dtype=np.int32)
        for i, r in enumerate(rows):
            idx[i, :len(r)] = r
        cnt = np.array([len(r) for r in rows], dtype=np.int32)
        bits = torch.empty((C, (T + 31) // 32), dtype=torch.int32, device="cuda")
        ws = torch.empty(lp.prefill_attn_dense_workspace(C, T, s.n_q, s.n_kv, s.d), dtype=torch.uint8, device="cuda")
        calls.append((q0, C, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(), bits, ws))

    def step():
        for q0, C, ti, tc, bits, ws in calls:
            T = q0 + C
            lp.fold_keep_bits(ti, tc, q0, T, s.fold_width, s.fold_recent, bits=bits)
            lp.prefill_attn_dense_bits(Q[q0:T], K[:T], V[:T], bits, s.scale, O=O[q0:T], workspace=ws)

    say("graph folded chunks")
    for o in [O] + [c[4] for c in calls]:
        o.fill_(float("nan") if o.is_floating_point() else -7)
    step()
    torch.cuda.synchronize()
    want = [O.clone().view(torch.int32)] + [c[4].clone() for c in calls]
    g = capture(step)
    other = torch.randn(1 << 20, device="cuda")
    replay_checks(g, [O] + [c[4] for c in calls], want, lambda: other.mul_(1.0001).sum())


def test_graph_blocksparse_chunks(lp):
    """A chunked block-sparse prefill (pooled index grown chunk by chunk, selection,
    block-sparse attention) over a 6,000-token prompt, whole in one graph."""
    rng = np.random.default_rng(5)
    N, n_q, n_kv, d, B, alpha = 6000, 8, 2, 128, 128, 0.1
    scale = float(np.float32(d ** -0.5))
    bits = lambda *sh: torch.from_numpy(rng.standard_normal(sh).astype(np.float32)).to(torch.bfloat16).cuda()
    Q, K, V = bits(N, n_q, d), bits(N, n_kv, d), bits(N, n_kv, d)
    nb = -(-N // B)
    kp = torch.empty((n_kv, nb, d), dtype=torch.float32, device="cuda")
    vp = torch.empty_like(kp)
    O = torch.empty((N, n_q, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(lp.prefill_attn_blocksparse_workspace(N, n_kv, d), dtype=torch.uint8, device="cuda")
    chunks = chunk_list(N, 2048)
    sel = []
    for q0, C in chunks:
        T = q0 + C
        nbT, nqb = -(-T // B), (T - 1) // B - q0 // B + 1
        sel.append((torch.empty((n_kv, nqb, nbT), dtype=torch.int32, device="cuda"),
                    torch.empty((n_kv, nqb), dtype=torch.int32, device="cuda")))

    def step():
        for (q0, C), (si, sc) in zip(chunks, sel):
            T = q0 + C
            lp.build_pooled_index(K[:T], V[:T], B, K_pool=kp, V_pool=vp, b_first=q0 // B)
            lp.select_blocks(Q[q0:T], kp, q0, B, alpha, scale, sel_idx=si, sel_cnt=sc)
            lp.prefill_attn_blocksparse(Q[q0:T], K[:T], V[:T], kp, vp, si, sc, q0, B, scale,
                                        O=O[q0:T], workspace=ws)

    say("graph block-sparse chunks")
    outs = [O, kp, vp] + [t for pair in sel for t in pair]
    for o in outs:   # the same fill as before each replay: parts no kernel writes compare equal
        o.fill_(float("nan") if o.is_floating_point() else -7)
    step()
    torch.cuda.synchronize()
    want = [o.clone().view(torch.int32) if o.is_floating_point() else o.clone() for o in outs]
    g = capture(step)
    other = torch.randn(1 << 20, device="cuda")
    replay_checks(g, outs, want, lambda: other.mul_(1.0001).sum())


def test_graph_gqa_chunks(lp):
    """gqa4k: the 4,096-row chunk and the 237-row tail (split key range and the
    combine) through the fp16-mask entry and the causal entry, in one graph."""
    from workloads import causal_mask
    w = make_workload("gqa4k")
    s = w.spec
    Q, K, V = dev_bf16(w.Q), dev_bf16(w.K), dev_bf16(w.V)
    O1 = torch.empty((w.N, s.n_q, s.d), dtype=torch.float32, device="cuda")
    O2 = torch.empty_like(O1)
    calls = []
    for q0, C in s.chunks:
        T = q0 + C
        ws = torch.empty(lp.prefill_attn_dense_workspace(C, T, s.n_q, s.n_kv, s.d), dtype=torch.uint8, device="cuda")
        calls.append((q0, C, torch.from_numpy(causal_mask(q0, C)).cuda(), ws))

    def step():
        for q0, C, mask, ws in calls:
            T = q0 + C
            lp.prefill_attn_dense(Q[q0:T], K[:T], V[:T], mask, s.scale, O=O1[q0:T], workspace=ws)
            lp.prefill_attn_dense_causal(Q[q0:T], K[:T], V[:T], q0, s.scale, O=O2[q0:T], workspace=ws)

    say("graph gqa chunks")
    for o in (O1, O2):
        o.fill_(float("nan"))
    step()
    torch.cuda.synchronize()
    want = [O1.clone().view(torch.int32), O2.clone().view(torch.int32)]
    g = capture(step)
    other = torch.randn(1 << 20, device="cuda")
    replay_checks(g, [O1, O2], want, lambda: other.mul_(1.0001).sum())
