#!/usr/bin/env python3
"""Prefill-attention benchmark on one MI355X.

Default workload "prefill32k" (Qwen3-4B attention shapes: 32 query heads,
8 KV heads, head_dim 128). One step is the whole hot path at 32K tokens:

  dense        the headline: the first 32,768 tokens of the seeded N(0,1) 128K
               prompt in 8 chunks of 4,096 rows, each over its accumulated
               history, under fp16 causal masks (mask-tile classification,
               fp16 value staging, tiled attention, split-key combine when
               needed);
  blocksparse  the planted 32K prompt: pooled index (block 128), alpha 0.1
               selection plus diagonal, exact attention on kept blocks with the
               pooled correction.

value = dense-equivalent FLOPs of the dense part (4*d*Hq*sum of visible keys,
8.796 TFLOP at 32K) / the dense part's time; tokens_per_s = 32,768 / that time;
pct_peak against the 2.5 PFLOP/s bf16 dense MFMA peak. The block-sparse part is
reported on its own: its time, the rate of the work it does (exact keys plus one
pooled row per skipped block) and its speedup over dense attention on the same
planted tensors (timed after the step loop, chunked and one-shot; the faster is
the comparator). Inputs are resident in HBM before timing starts. Also printed:
per-kernel times (HIP events recorded by the library on the launch stream), the
roofline of the dominant kernel and the fp64 CPU oracle timed on a bounded
sample of every workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 vector (256 CUs x 2.4 GHz x 256 FLOP per clock), published
METRIC = "prefill attention TFLOP/s (dense-equiv) + tokens/s at 32K; % bf16 MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill32k",
                    choices=["prefill32k", "dense128k", "sparse128k", "fold2k5", "gqa4k"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dense-entry", default="mask", choices=["mask", "causal", "bits", "gather"],
                    help="dense part: prefill_attn_dense over a causal fp16 mask (default), "
                         "prefill_attn_dense_causal (no mask buffer) or prefill_attn_dense_bits "
                         "(the same causal masks packed one bit per key); for the folded-selection "
                         "workload, mask (fold the lists, then dense), bits (fold the lists into keep "
                         "bits, then prefill_attn_dense_bits) or gather (prefill_attn_gather over the "
                         "lists)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="budget for the CPU oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 512 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--no-comparators", action="store_true",
                    help="skip the dense comparators on the block-sparse part's tensors")
    ap.add_argument("--parts", default="dense,blocksparse",
                    help="subset of the step to run (for profiler runs); the default runs the whole step")
    ap.add_argument("--graph", action="store_true",
                    help="time the step as HIP graph replays (one graph per part, captured after the "
                         "eager timed steps, which still give the per-kernel times): the launch cost of "
                         "the small prompts' many short kernels leaves the step")
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
    "stage_values": ("mask_combine.hip", "common.h"),
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    parts_sel = args.parts.split(",")

    def up_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # dense part: (workload, tokens, chunks); block-sparse part: (workload, calls)
    wd = ws_ = None
    if args.workload == "prefill32k":
        wd, Nd = make_workload("dense128k"), 32768          # the N(0,1) 128K prompt's first 32K tokens
        dchunks = chunk_list(Nd, 4096)
        ws_ = make_workload("sparse32k")
        scalls = ((0, ws_.N),)                               # one-shot over the planted prompt
    elif args.workload == "sparse128k":
        wd = ws_ = make_workload("sparse128k")
        Nd = wd.N
        dchunks = wd.spec.chunks
        scalls = wd.spec.chunks                              # chunked, incremental pooled index
    else:
        wd = make_workload(args.workload)
        Nd = wd.N
        dchunks = wd.spec.chunks
        scalls = ()
    do_dense = "dense" in parts_sel
    do_sparse = "blocksparse" in parts_sel and bool(scalls)
    s = wd.spec
    Hq, Hkv, d = s.n_q, s.n_kv, s.d
    scale = s.scale
    fold = args.workload == "fold2k5"

    Qd, Kd, Vd = up_bf16(wd.Q[:Nd]), up_bf16(wd.K[:Nd]), up_bf16(wd.V[:Nd])
    masks = [torch.from_numpy(causal_mask(q0, C)).to(dev) for q0, C in dchunks] if not fold else \
        [torch.empty((C, q0 + C), dtype=torch.float16, device=dev) for q0, C in dchunks]
    if args.dense_entry == "bits" and not fold:   # packed on the host before the timed region
        mask_bits = [torch.from_numpy(pack_keep_bits(causal_mask(q0, C) == 0)).to(dev) for q0, C in dchunks]
    if args.dense_entry == "bits" and fold:       # folded on the device inside each step
        mask_bits = [torch.empty((C, (q0 + C + 31) // 32), dtype=torch.int32, device=dev) for q0, C in dchunks]
    keeps = [fold_lists(wd, q0, C, dev) for q0, C in dchunks] if fold else []
    O_dense = torch.empty((Nd, Hq, d), dtype=torch.float32, device=dev)
    wsd = torch.empty(max(max(lp.prefill_attn_dense_workspace(C, q0 + C, Hq, Hkv, d) for q0, C in dchunks), 256),
                      dtype=torch.uint8, device=dev)

    if do_sparse:
        ss = ws_.spec
        B = ss.block
        Ns = ws_.N
        Qs, Ks, Vs = (Qd, Kd, Vd) if ws_ is wd else (up_bf16(ws_.Q), up_bf16(ws_.K), up_bf16(ws_.V))
        nb = -(-Ns // B)
        kp = torch.empty((Hkv, nb, d), dtype=torch.float32, device=dev)
        vp = torch.empty_like(kp)
        sel = []
        for q0, C in scalls:
            nbT, nq_blk = -(-(q0 + C) // B), (q0 + C - 1) // B - q0 // B + 1
            sel.append((torch.empty((Hkv, nq_blk, nbT), dtype=torch.int32, device=dev),
                        torch.empty((Hkv, nq_blk), dtype=torch.int32, device=dev)))
        O_sparse = torch.empty((Ns, Hq, d), dtype=torch.float32, device=dev)
        wss = torch.empty(max(lp.prefill_attn_blocksparse_workspace(Ns, Hkv, d), 256), dtype=torch.uint8,
                          device=dev)
    torch.cuda.synchronize()

    flops_dense = 4.0 * d * Hq * sum(dense_equiv_pairs(q0, C) for q0, C in dchunks)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def dense_call(Q, K, V, q0, C, ci, O, wsp, entry):
        T = q0 + C
        if keeps and entry == "gather":
            lp.prefill_attn_gather(Q[q0:T], K[:T], V[:T], keeps[ci][0], keeps[ci][1], q0, s.fold_width,
                                   s.fold_recent, scale, O=O[q0:T])
            return
        if keeps and entry == "bits":
            lp.fold_keep_bits(keeps[ci][0], keeps[ci][1], q0, T, s.fold_width, s.fold_recent, bits=mask_bits[ci])
        elif keeps:
            lp.fold_keep_mask(keeps[ci][0], keeps[ci][1], q0, T, s.fold_width, s.fold_recent, mask=masks[ci])
        if entry == "causal":
            lp.prefill_attn_dense_causal(Q[q0:T], K[:T], V[:T], q0, scale, O=O[q0:T], workspace=wsp)
        elif entry == "bits":
            lp.prefill_attn_dense_bits(Q[q0:T], K[:T], V[:T], mask_bits[ci], scale, O=O[q0:T], workspace=wsp)
        else:
            lp.prefill_attn_dense(Q[q0:T], K[:T], V[:T], masks[ci], scale, O=O[q0:T], workspace=wsp)

    kept_pairs = []
    if fold:   # (row, key) pairs the folded selection keeps, per chunk (for the gather roofline)
        for ci, (q0, C) in enumerate(dchunks):
            lp.fold_keep_mask(keeps[ci][0], keeps[ci][1], q0, q0 + C, s.fold_width, s.fold_recent,
                              mask=masks[ci])
            kept_pairs.append(int((masks[ci] == 0).sum().item()))
    if (args.dense_entry == "gather" and not fold) or (args.dense_entry == "causal" and fold):
        print("--dense-entry gather is for the folded-selection workload (fold2k5); causal is for "
              "causal workloads", file=sys.stderr)
        sys.exit(2)
    entry = args.dense_entry

    def run_dense():
        if do_dense:
            for ci, (q0, C) in enumerate(dchunks):
                dense_call(Qd, Kd, Vd, q0, C, ci, O_dense, wsd, entry)

    def run_sparse():
        # one pooled index for the whole prompt, pooled incrementally call by call
        for (q0, C), (si, sc) in zip(scalls, sel):
            T = q0 + C
            lp.build_pooled_index(Ks[:T], Vs[:T], B, K_pool=kp, V_pool=vp, b_first=q0 // B)
            lp.select_blocks(Qs[q0:T], kp, q0, B, ss.alpha, scale, sel_idx=si, sel_cnt=sc)
            lp.prefill_attn_blocksparse(Qs[q0:T], Ks[:T], Vs[:T], kp, vp, si, sc, q0, B, scale,
                                        O=O_sparse[q0:T], workspace=wss)

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

    dense_ms = float(np.median([a.elapsed_time(b) for a, b, _ in part_ev])) if do_dense else 0.0
    sparse_ms = float(np.median([b.elapsed_time(c) for _, b, c in part_ev])) if do_sparse else 0.0
    kern = {}
    for name in ("attn_dense", "mask_classify", "stage_values", "attn_combine", "attn_blocksparse", "pool",
                 "select", "fold", "attn_gather"):
        tot, n = lp.timing.read(name)
        if n:
            kern[name] = {"avg_ms": tot / n, "launches_per_step": n // args.steps, "ms_per_step": tot / args.steps}

    # graph replays: each part's launches captured once into a HIP graph (the
    # library allocates, synchronizes and clears nothing on its stream, so its
    # calls capture as they run), then K steps timed as replays
    eager = None
    if args.graph:
        graphs = {}
        for name, fn, on in (("dense", run_dense, do_dense), ("blocksparse", run_sparse, do_sparse)):
            if not on:
                continue
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            graphs[name] = g
        for g in graphs.values():
            g.replay()
        torch.cuda.synchronize()
        gev = []
        t0 = time.perf_counter()
        for _ in range(args.steps):
            e0, e1, e2 = ev(), ev(), ev()
            e0.record()
            if "dense" in graphs:
                graphs["dense"].replay()
            e1.record()
            if "blocksparse" in graphs:
                graphs["blocksparse"].replay()
            e2.record()
            gev.append((e0, e1, e2))
        torch.cuda.synchronize()
        eager = {"ms_per_step": round(ms_step, 4), "dense_ms": round(dense_ms, 4), "sparse_ms": round(sparse_ms, 4)}
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
        dense_ms = float(np.median([a.elapsed_time(b) for a, b, _ in gev])) if do_dense else 0.0
        sparse_ms = float(np.median([b.elapsed_time(c) for _, b, c in gev])) if do_sparse else 0.0

    # dense comparators on the block-sparse part's own tensors, timed after the
    # step loop (3 runs each, median): the same chunking as the block-sparse
    # calls' prompt in 4,096-row chunks, and (32K only) one call over the whole prompt
    comp = {}
    if do_sparse and not args.no_comparators:
        if ws_ is wd and do_dense:
            comp["chunked_ms"] = dense_ms
        else:
            cch = chunk_list(Ns, 4096)
            cm = [torch.from_numpy(causal_mask(q0, C)).to(dev) for q0, C in cch]
            O_c = torch.empty((Ns, Hq, d), dtype=torch.float32, device=dev)
            wsc = torch.empty(max(max(lp.prefill_attn_dense_workspace(C, q0 + C, Hq, Hkv, d) for q0, C in cch), 256),
                              dtype=torch.uint8, device=dev)

            def run_c():
                for (q0, C), m in zip(cch, cm):
                    T = q0 + C
                    lp.prefill_attn_dense(Qs[q0:T], Ks[:T], Vs[:T], m, scale, O=O_c[q0:T], workspace=wsc)
            comp["chunked_ms"] = time_median(run_c, ev, torch)
            del cm, wsc
            if len(scalls) == 1:
                r_ = torch.arange(Ns, device=dev)
                mask_full = torch.where(r_[None, :] <= r_[:, None], 0.0, -30000.0).to(torch.float16)
                del r_
                ws1 = torch.empty(max(lp.prefill_attn_dense_workspace(Ns, Ns, Hq, Hkv, d), 256),
                                  dtype=torch.uint8, device=dev)
                comp["oneshot_ms"] = time_median(
                    lambda: lp.prefill_attn_dense(Qs, Ks, Vs, mask_full, scale, O=O_c, workspace=ws1), ev, torch)
                del mask_full, ws1
            del O_c

    # HBM-bound kernels: algorithmic bytes per step / their event time per step
    hbm = {}
    if do_sparse and "pool" in kern:   # K and V of the tokens pooled (bf16) in, pooled rows (fp32) out
        hbm["pool"] = sum(2 * (q0 + C - (q0 // B) * B) * Hkv * d * 2 + 2 * (-(-(q0 + C) // B) - q0 // B) * Hkv * d * 4
                          for q0, C in scalls)
    if do_dense and "mask_classify" in kern and entry == "mask" and not fold:   # fp16 mask in, tile flags out
        hbm["mask_classify"] = sum(2 * C * (q0 + C) + (-(-C // 64)) * (-(-(q0 + C) // 64)) for q0, C in dchunks)
    if "stage_values" in kern:   # per call: V read twice (bf16: range pass, conversion), fp16 copy written
        calls = ([q0 + C for q0, C in dchunks] if do_dense else []) + \
                ([q0 + C for q0, C in scalls] if do_sparse else [])
        hbm["stage_values"] = sum(3 * T * Hkv * d * 2 for T in calls)
        if do_sparse:   # + the pooled operands of each block-sparse call: fp32 rows in, bf16/fp16 rows out
            hbm["stage_values"] += sum(-(-(q0 + C) // B) * Hkv * d * (2 * 4 + 2 * 2) for q0, C in scalls)
    hbm_kernels = {k: {"bytes_per_step": b, "GB_per_s": round(b / (kern[k]["ms_per_step"] * 1e-3) / 1e9, 1),
                       "frac_of_hbm_peak": round(b / (kern[k]["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                   for k, b in hbm.items()}

    parts = {}
    if do_dense:
        assert torch.isfinite(O_dense).all().item(), "non-finite dense output"
        parts["dense"] = {"ms": round(dense_ms, 3),
                          "tflops": round(flops_dense / (dense_ms * 1e-3) / 1e12, 2),
                          "pct_peak": round(100 * flops_dense / (dense_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                          "target_pct_peak": 50.0,
                          "tokens_per_s": round(Nd / (dense_ms * 1e-3)),
                          "data": f"{wd.spec.name} (seeded {'planted' if wd.spec.structure == 'planted' else 'N(0,1)'}"
                                  f"), first {Nd} tokens, {len(dchunks)} chunks"}
    if keeps and "fold" in kern:
        fold_bytes = sum(2 * C * (q0 + C) + 4 * keeps[i][0].numel() for i, (q0, C) in enumerate(dchunks))
        fold_ms = kern["fold"]["ms_per_step"]
        parts["fold"] = {"ms": round(fold_ms, 4), "GB_per_s": round(fold_bytes / (fold_ms * 1e-3) / 1e9, 1),
                         "bytes_per_step": fold_bytes, "hbm_peak_GB_per_s": 8000}
    if do_sparse:
        assert torch.isfinite(O_sparse).all().item(), "non-finite block-sparse output"
        visible = nb * (nb + 1) // 2 * Hkv   # the calls cover each query block once
        kept = sum(int(sc.sum().item()) for _, sc in sel)
        # the work the method does: exact keys of the kept blocks (the diagonal
        # causally) plus one pooled row per skipped visible block, 4 d FLOP per
        # (query head, row, key or pooled row)
        exact_flops = 4.0 * d * (Hq // Hkv) * sum(
            exact_pairs(sc.cpu().numpy(), q0, C, B) for (q0, C), (_, sc) in zip(scalls, sel))
        flops_sparse_equiv = 4.0 * d * Hq * sum(dense_equiv_pairs(q0, C) for q0, C in scalls)
        bs = {"ms": round(sparse_ms, 3), "workload": ws_.spec.name, "calls": len(scalls),
              "skipped_block_fraction": round(1.0 - kept / visible, 4),
              "exact_work_tflop": round(exact_flops / 1e12, 4),
              "exact_work_tflops": round(exact_flops / (sparse_ms * 1e-3) / 1e12, 2),
              "exact_work_pct_peak": round(100 * exact_flops / (sparse_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
              "tokens_per_s": round(Ns / (sparse_ms * 1e-3)),
              "dense_equiv_tflop": round(flops_sparse_equiv / 1e12, 4)}
        if "attn_blocksparse" in kern:
            kms = kern["attn_blocksparse"]["ms_per_step"]
            bs["attention_kernel_exact_work_tflops"] = round(exact_flops / (kms * 1e-3) / 1e12, 2)
        if comp:
            bs["dense_comparator_ms"] = {k: round(v, 3) for k, v in comp.items()}
            bs["speedup_vs_dense"] = round(min(comp.values()) / sparse_ms, 3)
        parts["blocksparse"] = bs

    # roofline of the dominant kernel: dense attention, algorithmic FLOPs per launch
    dom = "attn_dense" if do_dense else "attn_blocksparse"
    per_launch = flops_dense / len(dchunks) if do_dense else exact_flops / len(scalls)
    bound, peak = "mfma", PEAK_BF16_TFLOPS
    if entry == "gather":
        # fp32 VALU products over the kept keys only: 4 d FLOP per (query head, row, kept key)
        dom, bound, peak = "attn_gather", "alu", PEAK_FP32_TFLOPS
        per_launch = 4.0 * d * Hq * sum(kept_pairs) / len(dchunks)
        parts["dense"]["kept_pairs_per_head"] = int(sum(kept_pairs))
        parts["dense"]["kept_work_tflops"] = round(4.0 * d * Hq * sum(kept_pairs) / (dense_ms * 1e-3) / 1e12, 3)
    achieved = per_launch / (kern[dom]["avg_ms"] * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(dom, args.workload) if dom in KERNEL_SOURCES else None,
                "algorithmic_flops_per_launch": per_launch}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds)

    value = flops_dense / (dense_ms * 1e-3) / 1e12 if do_dense else exact_flops / (sparse_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1); planted block structure for the block-sparse part)",
        "config": {"workload": args.workload, "dense_entry": entry, "tokens": Nd, "n_q": Hq,
                   "n_kv": Hkv, "head_dim": d, "chunk": 4096 if args.workload != "fold2k5" else 1024,
                   "block": B if do_sparse else None, "alpha": ss.alpha if do_sparse else None,
                   "value_is": ("dense part: dense-equivalent FLOPs / its time" if do_dense else
                                "block-sparse exact work / its time"),
                   "step": ", then ".join(p for p, on in (
                       ("dense chunked prefill" + (" (indexer keep lists folded into the masks on the device)"
                                                   if fold else ""), do_dense),
                       ("block-sparse prefill" + (" in chunks (incremental pooled index)" if len(scalls) > 1 else ""),
                        do_sparse)) if on),
                   "parallelism": "none (1 GPU)",
                   "launch": "HIP graph replays (kernel times from the eager steps before them)" if args.graph
                             else "eager"},
        "tokens_per_s": round(Nd / (dense_ms * 1e-3)) if do_dense else round(Ns / (sparse_ms * 1e-3)),
        "pct_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "parts": parts, "kernels": kern, "roofline": roofline,
        "hbm_kernels": hbm_kernels, "cpu_baseline": cpu, "eager": eager,
        "device": {"name": props.name, "cus": props.multi_processor_count},
    }
    print(json.dumps(line), flush=True)


def time_median(fn, ev, torch, reps: int = 3) -> float:
    fn()
    ts = []
    for _ in range(reps):
        e0, e1 = ev(), ev()
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


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


def cpu_baseline(budget_s: float):
    """The fp64 oracle, as it stands, on a bounded sample of every workload.

    Each workload gets a slice of the time budget; what was run and the full
    oracle time it extrapolates to are reported per workload. The headline value
    is the dense oracle's dense-equivalent rate on the 32K headline's last chunk
    (4,096 rows over 32,768 keys), in the metric's unit."""
    from oracle import blocksparse_ref, dense_ref, pooled_index_ref, select_ref
    from workloads import bf16_to_f32, causal_mask, dense_equiv_pairs, make_workload

    def f64(b):
        return bf16_to_f32(b).astype(np.float64)

    per = {}
    t_all = time.perf_counter()

    # tiny, gqa4k, fold2k5: the whole dense oracle on every chunk
    for name in ("tiny", "gqa4k", "fold2k5"):
        w = make_workload(name)
        sp = w.spec
        t0 = time.perf_counter()
        pairs = 0
        for ci in range(len(sp.chunks)):
            q0, C, T, q, k, v, mask = w.chunk(ci)
            dense_ref(f64(q), f64(k), f64(v), mask, sp.scale)
            pairs += dense_equiv_pairs(q0, C)
        el = time.perf_counter() - t0
        fl = 4.0 * sp.d * sp.n_q * pairs
        per[name] = {"covered": "all chunks, all heads", "s": round(el, 2),
                     "tflops_dense_equiv": round(fl / el / 1e12, 5)}

    # the 32K dense headline: the last chunk (4,096 rows over 32K keys), heads until
    # the budget share runs out; the full 8-chunk oracle extrapolated from the rate
    w = make_workload("dense128k")
    sp = w.spec
    q0, C = 7 * 4096, 4096
    T = q0 + C
    q, k, v = f64(w.Q[q0:T]), f64(w.K[:T]), f64(w.V[:T])
    mask = causal_mask(q0, C)
    heads, fl = 0, 0.0
    t0 = time.perf_counter()
    for h in range(sp.n_q):
        dense_ref(q, k, v, mask, sp.scale, heads=[h])
        heads += 1
        fl += 4.0 * sp.d * dense_equiv_pairs(q0, C)
        if time.perf_counter() - t0 > 0.4 * budget_s:
            break
    el = time.perf_counter() - t0
    rate = fl / el
    full32 = 4.0 * sp.d * sp.n_q * sum(dense_equiv_pairs(4096 * c, 4096) for c in range(8))
    full128 = 4.0 * sp.d * sp.n_q * sum(dense_equiv_pairs(4096 * c, 4096) for c in range(32))
    per["dense32k"] = {"covered": f"chunk 7 (4,096 rows over 32,768 keys), {heads} of {sp.n_q} heads",
                       "s": round(el, 2), "tflops_dense_equiv": round(rate / 1e12, 5),
                       "extrapolated_full_s": round(full32 / rate, 1)}
    per["dense128k"] = {"covered": "extrapolated from the dense32k rate (same shapes)",
                        "extrapolated_full_s": round(full128 / rate, 1)}
    del q, k, v, mask

    # planted 32K block-sparse: the whole pooled index, the selection of a few query
    # blocks, the block-sparse oracle on rows of those blocks
    w = make_workload("sparse32k")
    sp = w.spec
    B = sp.block
    t0 = time.perf_counter()
    K64, V64 = f64(w.K), f64(w.V)
    kp, vp = pooled_index_ref(K64, V64, B)
    t_pool = time.perf_counter() - t0
    qb = [64, 128, 255]
    t1 = time.perf_counter()
    Q64 = f64(w.Q)
    from oracle import selection_sets
    sets = selection_sets(Q64, kp, 0, B, sp.alpha, sp.scale, qblocks=qb)
    t_sel = time.perf_counter() - t1
    nbk = sp.N // B
    ridx = np.zeros((sp.n_kv, nbk, nbk), dtype=np.int32)
    rcnt = np.zeros((sp.n_kv, nbk), dtype=np.int32)
    for (g, j), kept in sets.items():
        ridx[g, j, :len(kept)] = kept
        rcnt[g, j] = len(kept)
    rows = np.array([j * B + o for j in qb for o in (0, 127)])
    t2 = time.perf_counter()
    blocksparse_ref(Q64, K64, V64, kp, vp, ridx, rcnt, 0, B, sp.scale, rows=rows)
    t_att = time.perf_counter() - t2
    cand_done = sum(j for j in qb) * B * sp.n_q
    cand_all = sum(j for j in range(nbk)) * B * sp.n_q
    per["sparse32k"] = {"covered": f"pooled index whole ({t_pool:.1f} s); selection of query blocks {qb} "
                                   f"({t_sel:.1f} s); block-sparse oracle on {len(rows)} rows x all heads "
                                   f"({t_att:.1f} s)",
                        "s": round(t_pool + t_sel + t_att, 2),
                        "extrapolated_selection_full_s": round(t_sel * cand_all / cand_done, 1)}
    del select_ref
    total = time.perf_counter() - t_all
    return {"value": per["dense32k"]["tflops_dense_equiv"], "unit": "TFLOP/s", "cores": cpu_threads(),
            "cpu": cpu_model(), "kind": "oracle",
            "sample": "fp64 numpy oracle on the host's BLAS threads; value = dense oracle on the 32K "
                      "headline's last chunk; per-workload coverage and extrapolations in per_workload",
            "total_s": round(total, 1), "per_workload": per}


if __name__ == "__main__":
    main()
