#!/usr/bin/env python3
"""Throughput of the gfx950 attention path on one MI355X.

A step is one pass of the headline prefill workload: bf16 B=4, Hq=Hkv=16,
S=2048, D=64, run once with no mask and once causal (two attn_fwd launches on
inputs already resident in HBM).  The JSON line reports unmasked TFLOP/s
(4*D FLOPs per visible (query, key) pair) and the fraction of the 2.5 PFLOP/s
dense bf16 MFMA peak, the forward kernel's own launch times from HIP events,
the CPU oracle timed on a bounded sample of the same workload, and per-workload
figures for the other prefill shapes, the BlockMask build and the paged decode
(HBM GB/s against 8 TB/s).

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


class Timer:
    """HIP events on torch's current stream (the stream the kernels run on)."""

    def __init__(self, torch):
        self.torch = torch

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e


def bench_prefill(af, torch, workloads, w, steps, warmup, out_dtype=None, with_block_mask=None):
    dev = torch.device("cuda")
    inp = workloads.prefill_inputs(w)
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
        e0 = Timer(torch).event()
        for _ in range(10):
            af.attn_build_block_mask(w.mask, w.B, w.Sq, w.Skv, window=w.window,
                                     prefix_len=w.prefix_len, doc_ids=doc, device=dev, out=bm)
        e1 = Timer(torch).event()
        torch.cuda.synchronize()
        bm_us = e0.elapsed_time(e1) * 1000.0 / 10
    out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    kw = dict(scale=1.0 / math.sqrt(w.D), mask=w.mask, window=w.window, prefix_len=w.prefix_len,
              doc_ids=doc, score=w.score, softcap=w.softcap, block_mask=bm, out=out, lse=lse)
    for _ in range(warmup):
        af.attn_fwd(q, k, v, **kw)
    torch.cuda.synchronize()
    t = Timer(torch)
    e0 = t.event()
    for _ in range(steps):
        af.attn_fwd(q, k, v, **kw)
    e1 = t.event()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = visible_pairs(w.mask, w.Sq, w.window, inp["doc_lengths"])
    flops = 4.0 * w.D * w.B * w.Hq * pairs
    res = {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12, "gflop": flops / 1e9}
    res["frac_mfma_peak"] = res["tflops"] / MFMA_PEAK_TFLOPS
    if bm_us is not None:
        res["block_mask_build_us"] = bm_us
    return res


def bench_backward(af, torch, workloads, w, steps, warmup):
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
    for _ in range(warmup):
        af.attn_bwd(q, k, v, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
    torch.cuda.synchronize()
    t = Timer(torch)
    e0 = t.event()
    for _ in range(steps):
        af.attn_bwd(q, k, v, out, lse, do, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)
    e1 = t.event()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = visible_pairs(w.mask, w.Sq, w.window, inp["doc_lengths"])
    flops = 10.0 * w.D * w.B * w.Hq * pairs
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": ms, "tflops": tf, "gflop": flops / 1e9, "frac_mfma_peak": tf / MFMA_PEAK_TFLOPS}


def bench_decode(af, torch, workloads, steps, warmup, window=0, score="none"):
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
    for _ in range(warmup):
        af.attn_paged_decode(*args, **kw)
    torch.cuda.synchronize()
    t = Timer(torch)
    e0 = t.event()
    for _ in range(steps):
        af.attn_paged_decode(*args, **kw)
    e1 = t.event()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    lengths = [int(L) for L in inp["lengths"]]
    first = [max(0, L - window) if window else 0 for L in lengths]
    tokens = sum(L - t0 for L, t0 in zip(lengths, first))
    kv_bytes = tokens * 2 * w.Hkv * w.D * 2
    pages = sum(-(-L // w.page_size) - t0 // w.page_size for L, t0 in zip(lengths, first))
    algo_bytes = kv_bytes + n * hq * d * 2 * 2 + n * hq * 4 + pages * 4 + n * 4
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    return {"ms": ms, "GB_per_s": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS,
            "algorithmic_bytes": algo_bytes, "tokens": tokens}


def cpu_baseline(workloads, budget_s: float = 12.0):
    """The oracle, as it stands, on whole (batch, head) slices of the headline
    workload until about budget_s of CPU time is spent; rate on the same
    unmasked-FLOP basis."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    w_dense, w_causal = workloads.DENSE_BF16, workloads.CAUSAL_BF16
    q, k, v = workloads.randn_qkv(1, 1, 1, w_dense.Sq, w_dense.Skv, w_dense.D, "bf16", 0)
    qf = q.float().numpy().astype(np.float64)
    kf = k.float().numpy().astype(np.float64)
    vf = v.float().numpy().astype(np.float64)
    scale = 1.0 / math.sqrt(w_dense.D)
    flops = 0.0
    slices = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        oracle.attention_ref(qf, kf, vf, scale, oracle.MaskSpec(oracle.MASK_NONE))
        oracle.attention_ref(qf, kf, vf, scale, oracle.MaskSpec(oracle.MASK_CAUSAL))
        S = w_dense.Sq
        flops += 4.0 * w_dense.D * (S * S + S * (S + 1) // 2)
        slices += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{slices} x (one (batch, head) slice dense + one causal) of the "
                      f"B=4 H=16 S=2048 D=64 workload, float64 NumPy, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None,
                    help="run one workload (dense, causal, gqa, document, causal_softcap, "
                         "document_window, decode, decode_window, bwd_causal, bwd_dense, "
                         "bwd_gqa, bwd_document; for scale: long_dense_d128, "
                         "long_causal_d128, long_dense_d64) and exit")
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
            r = bench_backward(af, torch, workloads, wl, args.steps, args.warmup)
            print(json.dumps({"workload": args.only, **r}), flush=True)
            return
        if args.only == "decode":
            r = bench_decode(af, torch, workloads, args.steps, args.warmup)
        elif args.only == "decode_window":
            r = bench_decode(af, torch, workloads, args.steps, args.warmup, window=1024, score="alibi")
        else:
            r = bench_prefill(af, torch, workloads, sel[args.only], args.steps, args.warmup)
        print(json.dumps({"workload": args.only, **r}), flush=True)
        return

    # ---- headline: dense + causal prefill, bf16 B=4 H=16 S=2048 D=64
    dev = torch.device("cuda")
    wd, wc = workloads.DENSE_BF16, workloads.CAUSAL_BF16
    q, k, v = workloads.randn_qkv(wd.B, wd.Hq, wd.Hkv, wd.Sq, wd.Skv, wd.D, "bf16", 0)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    out_d = torch.empty_like(q)
    out_c = torch.empty_like(q)
    lse_d = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    lse_c = torch.empty_like(lse_d)
    scale = 1.0 / math.sqrt(wd.D)

    def dense():
        af.attn_fwd(q, k, v, scale=scale, mask="none", out=out_d, lse=lse_d)

    def causal():
        af.attn_fwd(q, k, v, scale=scale, mask="causal", out=out_c, lse=lse_c)

    for _ in range(args.warmup):
        dense()
        causal()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)
    t = Timer(torch)
    e0 = t.event()
    for _ in range(args.steps):
        dense()
        causal()
    e1 = t.event()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # Launch duration of each kernel variant: the same launch back to back
    # between two events on the launch stream, so the figure is the kernel's
    # own time (the launches queue ahead of the GPU).
    def launch_ms(fn):
        a0 = t.event()
        for _ in range(args.steps):
            fn()
        a1 = t.event()
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) / args.steps

    dense_ms = launch_ms(dense)
    causal_ms = launch_ms(causal)
    S = wd.Sq
    f_dense = 4.0 * wd.D * wd.B * wd.Hq * S * S
    f_causal = 4.0 * wd.D * wd.B * wd.Hq * S * (S + 1) // 2
    value = (f_dense + f_causal) / (ms_step * 1e-3) / 1e12
    kernel_ms = (dense_ms + causal_ms) / 2.0                     # mean launch duration
    achieved = ((f_dense + f_causal) / 2.0) / (kernel_ms * 1e-3) / 1e12
    src = os.path.join(ROOT, "attention_fa2_fwd_amd", "csrc", "fwd_bf16.hip")
    traffic = load_traffic(src, "fwd_bf16_d64_dense_causal")
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
        "config": {"workload": "dense_and_causal_prefill_bf16_b4_h16_s2048_d64",
                   "B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "S": S, "D": wd.D,
                   "masks": ["none", "causal"], "out_dtype": "bf16",
                   "flop_basis": "4*D per visible (query, key) pair"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                     "traffic": traffic, "kernel": "fwd_bf16_kernel<64, bf16 out>",
                     "launch_ms": {"dense": round(dense_ms, 5), "causal": round(causal_ms, 5)}},
        "cpu_baseline": None,
    }

    if not args.no_extra:
        extra = {}
        for name, w in (("gqa_window1024_alibi", workloads.GQA_WINDOW_ALIBI),
                        ("document_blockmask", workloads.DOCUMENT_BLOCKMASK),
                        ("causal_softcap5", workloads.CAUSAL_SOFTCAP),
                        ("document_window1024_blockmask", workloads.DOC_WINDOW_BLOCKMASK)):
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            extra[name] = bench_prefill(af, torch, workloads, w, 20, 3)
        for name, w in (("backward_causal_b4h16s2048d64", workloads.CAUSAL_BF16),
                        ("backward_gqa_window1024_alibi", workloads.GQA_WINDOW_ALIBI),
                        ("backward_document_blockmask", workloads.DOCUMENT_BLOCKMASK)):
            print(f"[bench] {name}", file=sys.stderr, flush=True)
            extra[name] = bench_backward(af, torch, workloads, w, 10, 2)
        print("[bench] paged decode", file=sys.stderr, flush=True)
        extra["paged_decode"] = bench_decode(af, torch, workloads, 20, 3)
        print("[bench] paged decode, window 1024 + alibi", file=sys.stderr, flush=True)
        extra["paged_decode_window1024_alibi"] = bench_decode(af, torch, workloads, 20, 3,
                                                              window=1024, score="alibi")
        line["workloads"] = {k2: {kk: (round(vv, 5) if isinstance(vv, float) else vv)
                                  for kk, vv in r.items()} for k2, r in extra.items()}
        line["workloads"]["dense_causal_split"] = {
            "dense_tflops": round(f_dense / (dense_ms * 1e-3) / 1e12, 3),
            "causal_tflops": round(f_causal / (causal_ms * 1e-3) / 1e12, 3)}

    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(workloads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
