#!/usr/bin/env python3
"""Throughput of the gfx950 attention path on one MI355X.

A step is one attn_fwd launch on the headline workload, the largest
single-GPU prefill configuration: bf16 GQA sliding window 1024 + ALiBi,
B=2, Hq=32, Hkv=8, S=8192, D=128, seed 0, inputs already resident in HBM.
The JSON line reports unmasked TFLOP/s (4*D FLOPs per visible (query, key)
pair) against the 2.5 PFLOP/s dense bf16 MFMA peak, with the forward kernel's
launch times (mean, median, min) from HIP events on the launch stream (after
0.3 s of back-to-back launches that bring the GPU to its steady clocks, then
the W counted warm-up steps); a
second roofline block for the paged decode of 64 sequences (HBM bytes
against 8 TB/s); the CPU oracle timed on (batch, head) slices of the
benchmarked tensors; and per-workload figures for the other prefill shapes,
the BlockMask build, the backward and the decode.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra]
                       [--no-cpu-baseline] [--only WORKLOAD] [--mode copy]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (unmasked) & % bf16 MFMA peak; decode HBM GB/s"
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def visible_pairs(mask: str, S: int, window: int = 0, doc_lengths=None) -> int:
    """Number of visible (query, key) pairs per (batch, head), square S x S."""
    if mask == "none":
        return S * S
    if mask == "causal":
        return S * (S + 1) // 2
    if mask == "sliding":
        w = window
        return sum(min(i + 1, w) for i in range(S))
    if mask == "document":
        return sum(n * (n + 1) // 2 for n in doc_lengths)
    if mask in ("sliding&document", "sliding&document&causal"):
        w = window
        return sum(n * (n + 1) // 2 if n <= w else w * (w + 1) // 2 + (n - w) * w
                   for n in doc_lengths)
    raise ValueError(mask)


def source_digest(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel_src: str, key: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel source has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(key)
    if not entry or entry.get("source_sha256_16") != source_digest(kernel_src):
        return None
    return entry.get("hbm_bytes_per_launch")


def time_launches(torch, fn, steps: int):
    """Run fn `steps` times back to back with a HIP event recorded on the
    launch stream (torch's current stream, where the binding enqueues) before
    the first launch and after each one.  Returns the mean over the whole
    run and the median and min of the per-launch intervals, in ms."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    mid = steps // 2
    median = per[mid] if steps % 2 else 0.5 * (per[mid - 1] + per[mid])
    return {"mean_ms": evs[0].elapsed_time(evs[steps]) / steps, "median_ms": median, "min_ms": per[0]}


PREWARM_S = 0.3   # seconds of back-to-back work before the counted warm-up steps


def prewarm(torch, fn, seconds: float = PREWARM_S) -> int:
    """Run fn back to back for about `seconds` of wall-clock time.  The GPU
    takes some tens of ms of continuous work to reach its steady clocks
    (launches of the GQA window workload run ~20% slower over the first
    ~20 ms); this runs before the W counted warm-up steps so that the K
    timed steps see the steady state.  Returns the launches run."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            fn()
        torch.cuda.synchronize()
        n += 16
    return n


def bench_prefill(af, torch, workloads, w, steps, warmup, out_dtype=None, with_block_mask=None,
                  inputs=None, prewarm_s: float = 0.0):
    """attn_fwd on a prefill workload; the BlockMask (when the workload has
    one) is built once, timed on its own and reused by every launch."""
    dev = torch.device("cuda")
    inp = workloads.prefill_inputs(w) if inputs is None else inputs
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    doc = inp["doc_ids"].to(dev) if inp["doc_ids"] is not None else None
    use_bm = w.block_mask if with_block_mask is None else with_block_mask
    bm = None
    bm_us = None
    if use_bm:
        for _ in range(3):
            bm = af.attn_build_block_mask(w.mask, w.B, w.Sq, w.Skv, window=w.window,
                                          prefix_len=w.prefix_len, doc_ids=doc, device=dev)
        torch.cuda.synchronize()
        # Builds into the same buffers, so the host issues them faster than
        # the kernel runs and the events time the kernels.
        t_bm = time_launches(torch, lambda: af.attn_build_block_mask(
            w.mask, w.B, w.Sq, w.Skv, window=w.window, prefix_len=w.prefix_len, doc_ids=doc,
            device=dev, out=bm), 10)
        bm_us = t_bm["mean_ms"] * 1000.0
    out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    kw = dict(scale=1.0 / math.sqrt(w.D), mask=w.mask, window=w.window, prefix_len=w.prefix_len,
              doc_ids=doc, score=w.score, softcap=w.softcap, block_mask=bm, out=out, lse=lse)
    if prewarm_s > 0:
        prewarm(torch, lambda: af.attn_fwd(q, k, v, **kw), prewarm_s)
    for _ in range(warmup):
        af.attn_fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    t = time_launches(torch, lambda: af.attn_fwd(q, k, v, **kw), steps)
    pairs = visible_pairs(w.mask, w.Sq, w.window, inp["doc_lengths"])
    flops = 4.0 * w.D * w.B * w.Hq * pairs
    ms = t["mean_ms"]
    res = {"ms": ms, "median_ms": t["median_ms"], "min_ms": t["min_ms"],
           "tflops": flops / (ms * 1e-3) / 1e12, "gflop": flops / 1e9}
    res["frac_mfma_peak"] = res["tflops"] / MFMA_PEAK_TFLOPS
    if bm_us is not None:
        res["block_mask_build_us"] = bm_us
    return res


def bench_backward(af, torch, workloads, w, steps, warmup, prewarm_s: float = 0.0):
    """attn_bwd on a prefill workload (its forward run once for O and LSE).
    Algorithmic FLOPs: 10 D per visible pair (the products S, dP, dV, dK,
    dQ: 2.5 times the forward's), whatever the kernels recompute."""
    dev = torch.device("cuda")
    inp = workloads.prefill_inputs(w)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    do = workloads.randn_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, w.dtype, w.seed + 1000)[0].to(dev)
    doc = inp["doc_ids"].to(dev) if inp["doc_ids"] is not None else None
    kw = dict(scale=1.0 / math.sqrt(w.D), mask=w.mask, window=w.window, prefix_len=w.prefix_len,
              doc_ids=doc, score=w.score, softcap=w.softcap)
    bm = None
    if w.block_mask:
        # built once and reused, as for the forward; the lists by key block too
        bm = af.attn_block_mask_transpose(
            af.attn_build_block_mask(w.mask, w.B, w.Sq, w.Skv, window=w.window, prefix_len=w.prefix_len,
                                     doc_ids=doc, device=dev))
    out, lse = af.attn_fwd(q, k, v, block_mask=bm, **kw)
    kw["block_mask"] = bm
    dq = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dk = torch.empty(k.shape, dtype=torch.float32, device=dev)
    dv = torch.empty(v.shape, dtype=torch.float32, device=dev)
    ws = torch.empty(max(int(af.load_library().attn_bwd_workspace_size(w.B, w.Hq, w.Sq)), 1),
                     dtype=torch.uint8, device=dev)
    if prewarm_s > 0:
        prewarm(torch, lambda: af.attn_bwd(q, k, v, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, **kw),
                prewarm_s)
    for _ in range(warmup):
        af.attn_bwd(q, k, v, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
    torch.cuda.synchronize()
    t = time_launches(torch, lambda: af.attn_bwd(q, k, v, out, lse, do, dq=dq, dk=dk, dv=dv,
                                                 workspace=ws, **kw), steps)
    ms = t["mean_ms"]
    pairs = visible_pairs(w.mask, w.Sq, w.window, inp["doc_lengths"])
    flops = 10.0 * w.D * w.B * w.Hq * pairs
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": ms, "median_ms": t["median_ms"], "min_ms": t["min_ms"], "tflops": tf,
            "gflop": flops / 1e9, "frac_mfma_peak": tf / MFMA_PEAK_TFLOPS}


def decode_algorithmic_bytes(w, lengths, window=0, hq=None):
    """Bytes the decode must move: each valid K/V byte once (per kv head),
    plus Q, O, LSE, the page ids of the pages read and seq_lens."""
    hq = w.Hq if hq is None else hq
    n = len(lengths)
    first = [max(0, L - window) if window else 0 for L in lengths]
    tokens = sum(L - t0 for L, t0 in zip(lengths, first))
    kv_bytes = tokens * 2 * w.Hkv * w.D * 2
    pages = sum(-(-L // w.page_size) - t0 // w.page_size for L, t0 in zip(lengths, first))
    return kv_bytes + n * hq * w.D * 2 * 2 + n * hq * 4 + pages * 4 + n * 4, tokens


def bench_decode(af, torch, workloads, steps, warmup, window=0, score="none", prewarm_s: float = 0.0):
    """Paged decode of the 64-sequence workload; with window > 0 each query
    sees its last `window` keys (and only those are counted as read)."""
    dev = torch.device("cuda")
    w = workloads.PAGED_DECODE
    inp = workloads.decode_inputs(w, device=dev)
    n, hq, d = inp["q"].shape
    need = af.attn_paged_decode_workspace_size(n, hq, d, w.max_pages)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp["q"])
    lse = torch.empty((n, hq), dtype=torch.float32, device=dev)
    args = (inp["q"], inp["k_cache"], inp["v_cache"], inp["page_table"], inp["seq_lens"])
    kw = dict(scale=1.0 / math.sqrt(d), workspace=ws, out=out, lse=lse,
              mask="sliding" if window else "none", window=window, score=score)
    if prewarm_s > 0:
        prewarm(torch, lambda: af.attn_paged_decode(*args, **kw), prewarm_s)
    for _ in range(warmup):
        af.attn_paged_decode(*args, **kw)
    torch.cuda.synchronize()
    t = time_launches(torch, lambda: af.attn_paged_decode(*args, **kw), steps)
    ms = t["mean_ms"]
    lengths = [int(L) for L in inp["lengths"]]
    algo_bytes, tokens = decode_algorithmic_bytes(w, lengths, window)
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    return {"ms": ms, "median_ms": t["median_ms"], "min_ms": t["min_ms"], "GB_per_s": gbs,
            "frac_hbm_peak": gbs / HBM_PEAK_GBS, "algorithmic_bytes": algo_bytes, "tokens": tokens}


def host_info():
    """CPU model, BLAS library and NumPy version of this host, and the BLAS
    thread count NumPy runs with."""
    import numpy as np
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info
        infos = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            blas = f"{infos[0].get('internal_api')} {infos[0].get('version')}"
            threads = max(int(i.get("num_threads", 1)) for i in infos)
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "blas": blas, "numpy": np.__version__, "threads": int(threads)}


def cpu_baseline(workloads, w, q, k, v, budget_s: float = 15.0):
    """The oracle, as it stands, on whole (batch, head) slices of the
    benchmarked tensors (the same bf16 values, read back as float64) until
    about budget_s of wall-clock time is spent; rate on the same
    unmasked-FLOP basis as the GPU figure (the oracle does the dense S x S
    work whatever the mask, so the rate is low by construction)."""
    import numpy as np
    import oracle
    info = host_info()
    scale = 1.0 / math.sqrt(w.D)
    ms = oracle.MaskSpec(workloads.MASK_NAMES[w.mask], window=w.window, prefix_len=w.prefix_len)
    ss = oracle.ScoreSpec(workloads.SCORE_NAMES[w.score])
    pairs = visible_pairs(w.mask, w.Sq, w.window)
    slices = []
    flops = 0.0
    t0 = time.perf_counter()
    for b in range(w.B):
        for hq in range(w.Hq):
            if time.perf_counter() - t0 >= budget_s:
                break
            hkv = hq * w.Hkv // w.Hq
            qs = q[b, hq].float().cpu().numpy().astype(np.float64)
            ks = k[b, hkv].float().cpu().numpy().astype(np.float64)
            vs = v[b, hkv].float().cpu().numpy().astype(np.float64)
            for r0 in range(0, w.Sq, 1024):
                rows = np.arange(r0, min(w.Sq, r0 + 1024))
                oracle.attention_rows(qs[rows], ks, vs, rows, b, hq, w.Hq, scale, ms, ss)
            flops += 4.0 * w.D * pairs
            slices.append((b, hq))
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": info["threads"], "kind": "oracle",
            "sample": f"{len(slices)} (batch, head) slices {slices[0]}..{slices[-1]} of the benchmarked "
                      f"{w.name} tensors, each its full {w.Sq} query rows against its kv head, "
                      f"float64 NumPy, {dt:.1f} s wall-clock (including the slices' host copies)",
            "seconds": round(dt, 3), "cpu_model": info["cpu_model"], "blas": info["blas"],
            "numpy": info["numpy"]}


ONLY = ("dense, causal, gqa, document, causal_softcap, document_window, decode, decode_window, "
        "bwd_causal, bwd_dense, bwd_gqa, bwd_document; for scale: long_dense_d128, "
        "long_causal_d128, long_dense_d64")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None, help=f"run one workload ({ONLY}) and exit")
    ap.add_argument("--mode", default="bench", choices=["bench", "copy"],
                    help="copy: a plain 1 GiB device copy, to calibrate byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; "
                                   f"--gpus {args.gpus} is not supported"}), flush=True)
        sys.exit(2)

    import torch
    import attention_fa2_fwd_amd as af
    import workloads
    af.load_library()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)

    if args.mode == "copy":
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": args.steps}), flush=True)
        return

    if args.only:
        sel = {"dense": workloads.DENSE_BF16, "causal": workloads.CAUSAL_BF16,
               "gqa": workloads.GQA_WINDOW_ALIBI, "document": workloads.DOCUMENT_BLOCKMASK,
               "causal_softcap": workloads.CAUSAL_SOFTCAP,
               "document_window": workloads.DOC_WINDOW_BLOCKMASK,
               "long_dense_d128": workloads.LONG_DENSE_D128,
               "long_causal_d128": workloads.LONG_CAUSAL_D128,
               "long_dense_d64": workloads.LONG_DENSE_D64}
        if args.only in ("bwd_causal", "bwd_gqa", "bwd_dense", "bwd_document"):
            wl = {"bwd_causal": workloads.CAUSAL_BF16, "bwd_gqa": workloads.GQA_WINDOW_ALIBI,
                  "bwd_dense": workloads.DENSE_BF16,
                  "bwd_document": workloads.DOCUMENT_BLOCKMASK}[args.only]
            r = bench_backward(af, torch, workloads, wl, args.steps, args.warmup, prewarm_s=PREWARM_S)
        elif args.only == "decode":
            r = bench_decode(af, torch, workloads, args.steps, args.warmup, prewarm_s=PREWARM_S)
        elif args.only == "decode_window":
            r = bench_decode(af, torch, workloads, args.steps, args.warmup, window=1024, score="alibi",
                             prewarm_s=PREWARM_S)
        elif args.only in sel:
            r = bench_prefill(af, torch, workloads, sel[args.only], args.steps, args.warmup,
                              prewarm_s=PREWARM_S)
        else:
            ap.error(f"--only takes one of: {ONLY}")
        print(json.dumps({"workload": args.only, **r}), flush=True)
        return

    # ---- headline: GQA sliding window 1024 + ALiBi, bf16 B=2 Hq=32 Hkv=8 S=8192 D=128
    dev = torch.device("cuda")
    w = workloads.GQA_WINDOW_ALIBI
    inp = workloads.prefill_inputs(w)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(w.D)

    def step():
        af.attn_fwd(q, k, v, scale=scale, mask=w.mask, window=w.window, score=w.score, out=out, lse=lse)

    prewarm_launches = prewarm(torch, step)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({prewarm_launches} pre-warm launches, {args.warmup} steps)",
          file=sys.stderr, flush=True)
    t = time_launches(torch, step, args.steps)     # synchronised on both sides
    ms_step = t["mean_ms"]
    pairs = visible_pairs(w.mask, w.Sq, w.window)
    flops = 4.0 * w.D * w.B * w.Hq * pairs
    value = flops / (ms_step * 1e-3) / 1e12
    src = os.path.join(ROOT, "attention_fa2_fwd_amd", "csrc", "fwd_bf16.hip")
    print(f"[bench] headline done: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gqa_sliding_window1024_alibi_prefill_bf16_b2_hq32_hkv8_s8192_d128",
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.Sq, "D": w.D, "mask": "sliding",
                   "window": w.window, "score": "alibi", "seed": w.seed, "out_dtype": "bf16",
                   "flop_basis": "4*D per visible (query, key) pair",
                   "visible_pairs_per_head": pairs},
        "roofline": {"bound": "mfma", "achieved": round(value, 3), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(value / MFMA_PEAK_TFLOPS, 4),
                     "traffic": load_traffic(src, "fwd_bf16_d128_gqa_window1024_alibi"),
                     "kernel": "fwd_bf16_kernel<128, SLIDING, bias, bf16 out>",
                     "flop_per_launch": flops,
                     "launch_ms": {"mean": round(t["mean_ms"], 5), "median": round(t["median_ms"], 5),
                                   "min": round(t["min_ms"], 5)},
                     "tflops_at_median": round(flops / (t["median_ms"] * 1e-3) / 1e12, 3)},
        "cpu_baseline": None,
        "prewarm": {"seconds": PREWARM_S, "launches": prewarm_launches,
                    "why": "the timed steps run at the GPU's steady clocks",
                    "other_workloads": f"each pre-warmed {PREWARM_S} s the same way"},
    }

    # ---- paged decode roofline (HBM), 64 sequences
    print("[bench] paged decode", file=sys.stderr, flush=True)
    dec = bench_decode(af, torch, workloads, 20, 3, prewarm_s=PREWARM_S)
    dsrc = os.path.join(ROOT, "attention_fa2_fwd_amd", "csrc", "decode.hip")
    line["roofline_decode"] = {
        "bound": "hbm", "achieved": round(dec["GB_per_s"], 3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(dec["frac_hbm_peak"], 4),
        "traffic": load_traffic(dsrc, "paged_decode_64seq"),
        "kernel": "decode_split_kernel + decode_combine_kernel (one attn_paged_decode call)",
        "workload": "paged_gqa_decode_bf16_n64_hq32_hkv8_d128_page16",
        "bytes_per_call": dec["algorithmic_bytes"],
        "call_ms": {"mean": round(dec["ms"], 5), "median": round(dec["median_ms"], 5),
                    "min": round(dec["min_ms"], 5)}}

    if not args.no_extra:
        extra = {}
        for name, wl in (("dense_b4h16s2048d64", workloads.DENSE_BF16),
                         ("causal_b4h16s2048d64", workloads.CAUSAL_BF16),
                         ("document_blockmask", workloads.DOCUMENT_BLOCKMASK),
                         ("causal_softcap5", workloads.CAUSAL_SOFTCAP),
                         ("document_window1024_blockmask", workloads.DOC_WINDOW_BLOCKMASK)):
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            extra[name] = bench_prefill(af, torch, workloads, wl, 20, 3, prewarm_s=PREWARM_S)
        for name, wl in (("backward_causal_b4h16s2048d64", workloads.CAUSAL_BF16),
                         ("backward_gqa_window1024_alibi", workloads.GQA_WINDOW_ALIBI),
                         ("backward_document_blockmask", workloads.DOCUMENT_BLOCKMASK)):
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            extra[name] = bench_backward(af, torch, workloads, wl, 10, 2, prewarm_s=PREWARM_S)
        extra["paged_decode"] = dec
        print("[bench] paged decode, window 1024 + alibi", file=sys.stderr, flush=True)
        extra["paged_decode_window1024_alibi"] = bench_decode(af, torch, workloads, 20, 3,
                                                              window=1024, score="alibi",
                                                              prewarm_s=PREWARM_S)
        line["workloads"] = {k2: {kk: (round(vv, 5) if isinstance(vv, float) else vv)
                                  for kk, vv in r.items()} for k2, r in extra.items()}

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(workloads, w, q, k, v)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
