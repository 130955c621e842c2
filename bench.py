#!/usr/bin/env python3
"""Prefill-attention benchmark on one MI355X.

Default workload "prefill32k" (Qwen3-4B attention shapes: 32 query heads,
8 KV heads, head_dim 128, 32,768 tokens, planted synthetic Q/K/V). One step is
the whole hot path over that prompt, done both ways on the same tensors:

  dense        8 chunks of 4,096 rows, each over its accumulated history, under
               an fp16 causal mask (mask-tile classification, tiled attention,
               split-key combine when needed);
  blocksparse  pooled index (block 128), alpha 0.1 selection plus diagonal,
               exact attention on kept blocks with the pooled correction.

value = dense-equivalent FLOPs of the step (2 x 4*d*Hq*N(N+1)/2) / step time.
Inputs are resident in HBM before timing starts. Also printed: per-part
TFLOP/s, tokens/s and % of the bf16 dense MFMA peak, the roofline of the
dominant kernel (HIP events around each of its launches, on its stream), and
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
METRIC = "prefill attention TFLOP/s (dense-equiv) + tokens/s at 32K; % bf16 MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill32k",
                    choices=["prefill32k", "dense128k", "sparse128k", "fold2k5", "gqa4k"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dense-entry", default="mask", choices=["mask", "causal", "bits"],
                    help="dense part: prefill_attn_dense over a causal fp16 mask (default), "
                         "prefill_attn_dense_causal (no mask buffer) or prefill_attn_dense_bits "
                         "(the same causal masks packed one bit per key)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the CPU oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 512 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--no-oneshot", action="store_true",
                    help="skip the one-shot dense comparator (one call over the whole 32K prompt)")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the register-only MFMA calibration (random vs zero bf16 operands)")
    ap.add_argument("--parts", default="dense,blocksparse",
                    help="subset of the step to run (for profiler runs); the default runs the whole step")
    return ap.parse_args()


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_prefill_attn_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# sources each timed kernel is built from (a counter record is valid for one version)
KERNEL_SOURCES = {
    "attn_dense": ("attention.hip", "common.h"),
    "attn_blocksparse": ("attention.hip", "common.h"),
    "attn_combine": ("mask_combine.hip", "common.h"),
    "mask_classify": ("mask_combine.hip", "common.h"),
    "pool": ("pool_select.hip", "common.h"),
    "select": ("pool_select.hip", "common.h"),
}


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(f"{kernel}:{workload}")
    if not rec or rec.get("source_sha") != source_hash(*KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path is built and timed on a single MI355X. "
              "Sharding across GPUs (by KV head, or by key range with an LSE merge) is not built. "
              "Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_prefill_attn_amd as lp
    from workloads import causal_mask, dense_equiv_pairs, make_workload, pack_keep_bits
    from workloads.gen import chunk_list

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    def up_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # prefill32k: dense in 4,096-row chunks + one-shot block-sparse of the same 32K prompt
    # sparse128k: dense and block-sparse, both in 4,096-row chunks over the growing history
    # dense128k: dense in 4,096-row chunks only
    chunked_sparse = args.workload == "sparse128k"
    if args.workload == "prefill32k":
        w = make_workload("sparse32k")
        chunks = chunk_list(w.N, 4096)
        do_sparse = "blocksparse" in args.parts.split(",")
    elif args.workload == "sparse128k":
        w = make_workload("sparse128k")
        chunks = w.spec.chunks
        do_sparse = "blocksparse" in args.parts.split(",")
    elif args.workload == "gqa4k":
        # the ~4,333-token prompt: chunk 4,096 at history 0, then the 237-row tail
        # chunk over the 4,096-token history (16 query heads, 4 KV heads)
        w = make_workload("gqa4k")
        chunks = w.spec.chunks
        do_sparse = False
    elif args.workload == "fold2k5":
        # the ~2,500-token narrow-chunk prompt; each step folds the indexer's keep
        # lists into the chunk masks on the device, then runs dense attention
        w = make_workload("fold2k5")
        chunks = w.spec.chunks
        do_sparse = False
    else:
        w = make_workload("dense128k")
        chunks = w.spec.chunks
        do_sparse = False
    s = w.spec
    N, Hq, Hkv, d, B = w.N, s.n_q, s.n_kv, s.d, s.block
    scale = s.scale

    Q, K, V = up_bf16(w.Q), up_bf16(w.K), up_bf16(w.V)
    masks = [torch.from_numpy(causal_mask(q0, C)).to(dev) for q0, C in chunks]
    if args.dense_entry == "bits":   # packed on the host before the timed region
        mask_bits = [torch.from_numpy(pack_keep_bits(causal_mask(q0, C) == 0)).to(dev) for q0, C in chunks]
    keeps = [fold_lists(w, q0, C, dev) for q0, C in chunks] if args.workload == "fold2k5" else []
    O_dense = torch.empty((N, Hq, d), dtype=torch.float32, device=dev)
    ws_bytes = max(lp.prefill_attn_dense_workspace(C, q0 + C, Hq, Hkv, d) for q0, C in chunks)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    nb = -(-N // B)
    kp = torch.empty((Hkv, nb, d), dtype=torch.float32, device=dev)
    vp = torch.empty_like(kp)
    sparse_calls = [(q0, C) for q0, C in chunks] if chunked_sparse else [(0, N)]
    sel = []   # per call: (sel_idx, sel_cnt)
    for q0, C in sparse_calls if do_sparse else []:
        nbT, nq_blk = -(-(q0 + C) // B), (q0 + C - 1) // B - q0 // B + 1
        sel.append((torch.empty((Hkv, nq_blk, nbT), dtype=torch.int32, device=dev),
                    torch.empty((Hkv, nq_blk), dtype=torch.int32, device=dev)))
    O_sparse = torch.empty((N, Hq, d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    run_dense_part = "dense" in args.parts.split(",")
    pairs = sum(dense_equiv_pairs(q0, C) for q0, C in chunks)
    flops_dense = 4.0 * d * Hq * pairs if run_dense_part else 0.0
    flops_sparse = 4.0 * d * Hq * dense_equiv_pairs(0, N) if do_sparse else 0.0

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def run_dense():
        if not run_dense_part:
            return
        for ci, ((q0, C), m) in enumerate(zip(chunks, masks)):
            T = q0 + C
            if keeps:
                lp.fold_keep_mask(keeps[ci][0], keeps[ci][1], q0, T, s.fold_width, s.fold_recent, mask=m)
            if args.dense_entry == "causal" and not keeps:
                lp.prefill_attn_dense_causal(Q[q0:T], K[:T], V[:T], q0, scale, O=O_dense[q0:T], workspace=ws)
            elif args.dense_entry == "bits" and not keeps:
                lp.prefill_attn_dense_bits(Q[q0:T], K[:T], V[:T], mask_bits[ci], scale, O=O_dense[q0:T],
                                           workspace=ws)
            else:
                lp.prefill_attn_dense(Q[q0:T], K[:T], V[:T], m, scale, O=O_dense[q0:T], workspace=ws)

    def run_sparse():
        # one pooled index for the whole prompt, pooled incrementally chunk by chunk
        for (q0, C), (si, sc) in zip(sparse_calls, sel):
            T = q0 + C
            lp.build_pooled_index(K[:T], V[:T], B, K_pool=kp, V_pool=vp, b_first=q0 // B)
            lp.select_blocks(Q[q0:T], kp, q0, B, s.alpha, scale, sel_idx=si, sel_cnt=sc)
            lp.prefill_attn_blocksparse(Q[q0:T], K[:T], V[:T], kp, vp, si, sc, q0, B, scale,
                                        O=O_sparse[q0:T])

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        run_dense()
        if do_sparse:
            run_sparse()
    torch.cuda.synchronize()

    lp.timing.reset()
    lp.timing.enable(True)
    part_ev = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e0, e1, e2 = ev(), ev(), ev()
        e0.record()
        run_dense()
        e1.record()
        if do_sparse:
            run_sparse()
        e2.record()
        part_ev.append((e0, e1, e2))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    lp.timing.enable(False)

    ms_step = wall * 1e3 / args.steps

    # the one-shot dense comparator for the block-sparse half (one call over the
    # whole prompt under its causal mask), timed after the step loop
    oneshot_ms = None
    if do_sparse and run_dense_part and not chunked_sparse and not args.no_oneshot:
        r_ = torch.arange(N, device=dev)
        mask_full = torch.where(r_[None, :] <= r_[:, None], 0.0, -30000.0).to(torch.float16)
        del r_
        ws1 = torch.empty(max(lp.prefill_attn_dense_workspace(N, N, Hq, Hkv, d), 256), dtype=torch.uint8,
                          device=dev)
        lp.prefill_attn_dense(Q, K, V, mask_full, scale, O=O_dense, workspace=ws1)
        ts = []
        for _ in range(3):
            e0, e1 = ev(), ev()
            e0.record()
            lp.prefill_attn_dense(Q, K, V, mask_full, scale, O=O_dense, workspace=ws1)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        oneshot_ms = float(np.median(ts))
        del mask_full, ws1
    dense_ms = float(np.median([a.elapsed_time(b) for a, b, _ in part_ev]))
    sparse_ms = float(np.median([b.elapsed_time(c) for _, b, c in part_ev])) if do_sparse else 0.0
    kern = {}
    for name in ("attn_dense", "mask_classify", "attn_combine", "attn_blocksparse", "pool", "select", "fold"):
        tot, n = lp.timing.read(name)
        if n:
            kern[name] = {"avg_ms": tot / n, "launches_per_step": n // args.steps, "ms_per_step": tot / args.steps}

    # HBM-bound kernels: algorithmic bytes per step / their event time per step
    hbm = {}
    if "pool" in kern:   # K and V of the tokens pooled (bf16) in, pooled rows (fp32) out
        pool_bytes = sum(2 * (q0 + C - (q0 // B) * B) * Hkv * d * 2 + 2 * (-(-(q0 + C) // B) - q0 // B) * Hkv * d * 4
                         for q0, C in sparse_calls)
        hbm["pool"] = pool_bytes
    if "mask_classify" in kern and args.dense_entry == "mask" and not keeps:   # fp16 mask in, tile flags out
        hbm["mask_classify"] = sum(2 * C * (q0 + C) + (-(-C // 128)) * (-(-(q0 + C) // 128)) for q0, C in chunks)
    hbm_kernels = {k: {"bytes_per_step": b, "GB_per_s": round(b / (kern[k]["ms_per_step"] * 1e-3) / 1e9, 1),
                       "frac_of_hbm_peak": round(b / (kern[k]["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                   for k, b in hbm.items()}

    assert torch.isfinite(O_dense).all().item(), "non-finite dense output"
    if do_sparse:
        assert torch.isfinite(O_sparse).all().item(), "non-finite block-sparse output"
        visible = nb * (nb + 1) // 2 * Hkv   # chunks cover each query block once (4,096 = 32 B)
        kept = sum(int(sc.sum().item()) for _, sc in sel)
        sparsity = 1.0 - kept / visible
        # the work the method does: exact keys of the kept blocks (the diagonal
        # causally) plus one pooled row per skipped visible block, 4 d FLOP per
        # (query head, row, key or pooled row)
        exact_flops = 4.0 * d * (Hq // Hkv) * sum(
            exact_pairs(sc.cpu().numpy(), q0, C, B) for (q0, C), (_, sc) in zip(sparse_calls, sel))
    tflops = (flops_dense + flops_sparse) / (ms_step * 1e-3) / 1e12

    # roofline of the dominant kernel: dense attention, algorithmic FLOPs per launch
    dom = "attn_dense" if run_dense_part else "attn_blocksparse"
    per_launch_flops = flops_dense / len(chunks) if run_dense_part else flops_sparse
    achieved = per_launch_flops / (kern[dom]["avg_ms"] * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom, args.workload),
                "algorithmic_flops_per_launch": per_launch_flops}

    parts = {}
    if run_dense_part:
        parts["dense"] = {"ms": round(dense_ms, 3),
                          "tflops": round(flops_dense / (dense_ms * 1e-3) / 1e12, 2),
                          "pct_peak": round(100 * flops_dense / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                          "tokens_per_s": round(N / (dense_ms * 1e-3))}
    if keeps:
        fold_bytes = sum(2 * C * (q0 + C) + 4 * keeps[i][0].numel() for i, (q0, C) in enumerate(chunks))
        fold_ms = kern["fold"]["ms_per_step"]
        parts["fold"] = {"ms": round(fold_ms, 4), "GB_per_s": round(fold_bytes / (fold_ms * 1e-3) / 1e9, 1),
                         "bytes_per_step": fold_bytes, "hbm_peak_GB_per_s": 8000}
    if do_sparse:
        parts["blocksparse"] = {"ms": round(sparse_ms, 3),
                                "tflops_dense_equiv": round(flops_sparse / (sparse_ms * 1e-3) / 1e12, 2),
                                "pct_peak_dense_equiv": round(100 * flops_sparse / (sparse_ms * 1e-3) / 1e12
                                                              / PEAK_BF16_TFLOPS, 2),
                                "tokens_per_s": round(N / (sparse_ms * 1e-3)),
                                "skipped_block_fraction": round(sparsity, 4),
                                "exact_work_tflops": round(exact_flops / (sparse_ms * 1e-3) / 1e12, 2),
                                "exact_work_pct_peak": round(100 * exact_flops / (sparse_ms * 1e-3) / 1e12
                                                             / PEAK_BF16_TFLOPS, 2),
                                "speedup_vs_dense": round(dense_ms / sparse_ms, 3) if run_dense_part else None}
        if oneshot_ms is not None:
            parts["dense_oneshot"] = {"ms": round(oneshot_ms, 3),
                                      "tflops": round(flops_sparse / (oneshot_ms * 1e-3) / 1e12, 2),
                                      "pct_peak": round(100 * flops_sparse / (oneshot_ms * 1e-3) / 1e12
                                                        / PEAK_BF16_TFLOPS, 2)}
            parts["blocksparse"]["speedup_vs_oneshot_dense"] = round(oneshot_ms / sparse_ms, 3)
            parts["blocksparse"]["speedup_vs_faster_dense"] = round(min(oneshot_ms, dense_ms) / sparse_ms, 3)

    ceiling = None if args.no_mfma_ceiling else mfma_ceiling(lp, torch, dev, props.multi_processor_count)
    if ceiling:
        roofline["frac_of_random_operand_mfma_rate"] = round(achieved / ceiling["random_bf16_tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, chunks, args.cpu_seconds)

    line = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; planted block structure)" if do_sparse else "synthetic (seeded N(0,1))",
        "config": {"workload": args.workload, "dense_entry": args.dense_entry, "tokens": N, "n_q": Hq,
                   "n_kv": Hkv, "head_dim": d,
                   "chunk": 4096, "block": B if do_sparse else None,
                   "alpha": s.alpha if do_sparse else None,
                   "step": ("dense chunked + chunked block-sparse (incremental pooled index) prefill of "
                            "the same prompt" if chunked_sparse else
                            "dense chunked + block-sparse prefill of the same prompt") if do_sparse
                   else ("indexer keep lists folded into the masks on the device + dense chunked prefill"
                         if keeps else "dense chunked prefill"), "parallelism": "none (1 GPU)"},
        "tokens_per_s": round((2 if do_sparse else 1) * N / (ms_step * 1e-3)),
        "pct_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "parts": parts, "kernels": kern, "roofline": roofline, "mfma_ceiling": ceiling,
        "hbm_kernels": hbm_kernels, "cpu_baseline": cpu,
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    print(json.dumps(line), flush=True)


def exact_pairs(cnt, q0, C, B):
    """(row, key) pairs one query head computes in a block-sparse call, pooled
    rows counted as one key each: for query block j with c kept blocks (the
    diagonal included) and rows [rlo, rhi) of the call, rows x (c - 1) x B exact
    keys, the diagonal's causal keys, and rows x (j - (c - 1)) pooled rows;
    summed over the KV heads (cnt is [n_kv][n_qblk])."""
    total = 0
    j0 = q0 // B
    for jj in range(cnt.shape[1]):
        j = j0 + jj
        rlo, rhi = max(j * B, q0), min((j + 1) * B, q0 + C)
        rows = rhi - rlo
        diag = sum(p - j * B + 1 for p in range(rlo, rhi))
        c = cnt[:, jj].astype(np.int64)
        total += int((rows * (c - 1) * B + diag + rows * (j - (c - 1))).sum())
    return total


def mfma_ceiling(lp, torch, dev, cus):
    """bf16 MFMA rate sustained from registers (pa_mfma_probe) with random N(0,1)
    bf16 operands, as the attention kernels see, and with zero operands; best of
    three ~30 ms runs each, after the timed region. The gap between the two is
    the clock the matrix cores' operand-dependent power draw costs."""
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    rnd = torch.randn(1 << 19, device=dev, generator=g).to(torch.bfloat16)   # 1 MiB
    zero = torch.zeros_like(rnd)
    sink = torch.empty(4 * cus * 512, dtype=torch.float32, device=dev)
    iters = 6000
    flops = 4 * cus * 8 * iters * 32 * 32768.0
    out = {}
    for name, ops, shape in (("random_bf16_tflops", rnd, 32), ("zero_tflops", zero, 32),
                             ("random_bf16_16x16x32_tflops", rnd, 16)):
        lp.mfma_probe(ops, sink, 200, shape)
        best = float("inf")
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            lp.mfma_probe(ops, sink, iters, shape)
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        out[name] = round(flops / (best * 1e-3) / 1e12, 1)
    out["random_frac_of_peak"] = round(out["random_bf16_tflops"] / PEAK_BF16_TFLOPS, 4)
    out["probe"] = (f"{4 * cus} workgroups x 8 waves, {iters} x 32 v_mfma_f32_32x32x16_bf16 (the attention "
                    "kernels' shape; 4 accumulators) or the same FLOPs as 16x16x32 (8 accumulators) per "
                    "wave, from registers")
    return out


def fold_lists(w, q0, C, dev):
    """Compacted keep lists (blocks of fold_width keys) of the chunk's rows, as a
    sparse indexer would return them: every block up to the row while the row
    sees at most the budget, else the drawn blocks (the recent keys are added by
    the fold itself)."""
    import torch
    s = w.spec
    rows = [list(range(p // s.fold_width + 1)) if p + 1 <= s.fold_budget
            else [int(c) for c in w.keep_blocks[p]] for p in range(q0, q0 + C)]
    idx = np.zeros((C, max(len(r) for r in rows)), dtype=np.int32)
    for i, r in enumerate(rows):
        idx[i, :len(r)] = r
    cnt = np.array([len(r) for r in rows], dtype=np.int32)
    return torch.from_numpy(idx).to(dev), torch.from_numpy(cnt).to(dev)


def cpu_baseline(w, chunks, budget_s):
    """The fp64 oracle on a bounded sample: the last 4,096-row chunk of the dense
    pass (all 32K keys), as many query heads as fit in the time budget."""
    from oracle import dense_ref
    from workloads import bf16_to_f32, causal_mask
    s = w.spec
    q0, C = chunks[-1]
    T = q0 + C
    q = bf16_to_f32(w.Q[q0:T]).astype(np.float64)
    k = bf16_to_f32(w.K[:T]).astype(np.float64)
    v = bf16_to_f32(w.V[:T]).astype(np.float64)
    mask = causal_mask(q0, C)
    heads = 0
    flops = 0.0
    t0 = time.perf_counter()
    for h in range(s.n_q):
        dense_ref(q, k, v, mask, s.scale, heads=[h])
        heads += 1
        flops += 4.0 * s.d * (C * q0 + C * (C + 1) / 2)
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(flops / el / 1e12, 5), "unit": "TFLOP/s", "cores": cpu_threads(),
            "kind": "oracle",
            "sample": f"dense oracle (fp64 numpy) on chunk {len(chunks) - 1} ({C} rows over {T} keys), "
                      f"{heads} of {s.n_q} query heads, {el:.1f} s"}


if __name__ == "__main__":
    main()
