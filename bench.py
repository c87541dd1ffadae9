"""Benchmark of the block-sparse paged attention path on one MI355X.

One step = one bsr_run_decode call on the batch-64 paged decode workload (bf16,
KV lengths U[512, 8192], page size 16, 32 query / 8 KV heads, head_dim 128): the
attention kernel over the planned split-KV partition plus the merge of the partial
states.  The plan is built once and reused by every step (it is per generation step
and shared by all layers).  Inputs are resident in HBM before timing; three copies of
the KV pool are rotated so the last-level cache cannot serve a step from the previous
one.  The same JSON line also reports the ragged causal prefill (TFLOP/s), the
vector-sparse (page size 1) runs next to their contiguous twins, the composable
shared-prefix decode, the roofline of the dominant kernel, and the fp64 CPU oracle
timed on a bounded sample as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "paged decode HBM GB/s (% of peak); causal prefill TFLOPS (% bf16 MFMA peak)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(kv_lens, B, Hq, Hk, d, nnz, elt=2):
    """Algorithmic bytes of one decode call: K and V read once, Q read, O and LSE written,
    plus the page table (indices, indptr, last-page lengths)."""
    kv = int(np.sum(kv_lens)) * Hk * d * elt * 2
    qo = 2 * B * Hq * d * elt
    return kv + qo + B * Hq * 4 + nnz * 4 + (B + 1) * 4 + B * 4


def prefill_flops(lens, Hq, d):
    """QK^T and PV flops over the unmasked (causal) pairs only."""
    return float(sum(4.0 * d * Hq * l * (l + 1) / 2 for l in lens))


def time_calls(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(steps):
        fn(s)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def per_call_ms(fn, n):
    """Median / min / p90 of individually event-timed calls."""
    import torch

    ts = []
    for s in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(s)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    ts = np.array(ts)
    return float(np.median(ts)), float(ts.min()), float(np.percentile(ts, 90))


def kernel_times(fn, n):
    """Average per-launch durations of the attention and merge kernels, measured with HIP
    events that the library records on the launch stream around each kernel."""
    import torch
    from block_sparse_paged_bsr_amd import api

    torch.cuda.synchronize()
    api.timing_enable(True)
    for s in range(n):
        fn(s)
    t = api.timing_read()
    api.timing_enable(False)
    return (t["attn_ms"] / max(t["attn_launches"], 1), t["attn_launches"],
            t["merge_ms"] / max(t["merge_launches"], 1), t["merge_launches"])


def bench_decode(args):
    import torch
    from block_sparse_paged_bsr_amd import api, inputs

    b = inputs.batched_decode_bf16(seed=0, poison=False)
    q, k, v = b.torch_values("cuda")
    C = api.query_num_workers("decode", 32, 8, 128)
    t0 = time.perf_counter()
    p = api.Plan(b.kv_indptr, b.kv_indices, b.last_page_len, num_pages=b.num_pages, num_qo_heads=32,
                 num_kv_heads=8, head_dim=128, page_size=16, num_workers=C)
    plan_us = (time.perf_counter() - t0) * 1e6
    ws = api.alloc_workspace(p)
    p.upload(ws)
    pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(2)]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], 32, dtype=torch.float32, device="cuda")
    sm = 1.0 / math.sqrt(128)

    def step(s):
        kk, vv = pools[s % len(pools)]
        api.run_decode(p, ws, q, kk, vv, o=o, lse=lse, sm_scale=sm)

    ms = time_calls(step, args.steps, args.warmup)
    med, mn, p90 = per_call_ms(step, 50)
    attn_ms, n_attn, merge_ms, n_merge = kernel_times(step, 50)
    nbytes = decode_bytes(b.kv_lens, b.batch, 32, 8, 128, len(b.kv_indices))
    e = p.export()
    return {
        "ms_per_step": ms,
        "gbs": nbytes / (ms * 1e-3) / 1e9,
        "bytes": nbytes,
        "median_ms": med, "min_ms": mn, "p90_ms": p90,
        "attn_kernel_ms": attn_ms, "merge_kernel_ms": merge_ms,
        "attn_launches": n_attn, "merge_launches": n_merge,
        "plan_host_us": plan_us, "num_workers": C, "num_items": int(e["items"].shape[0]),
        "num_slots": e["num_slots"], "tokens": int(b.kv_lens.sum()), "batch": b,
    }


def bench_prefill(args):
    import torch
    from block_sparse_paged_bsr_amd import api, inputs

    b = inputs.ragged_prefill_bf16(seed=0, poison=False)
    q, k, v = b.torch_values("cuda")
    C = api.query_num_workers("prefill", 32, 8, 128)
    p = api.Plan(b.kv_indptr, b.kv_indices, b.last_page_len, num_pages=b.num_pages, num_qo_heads=32,
                 num_kv_heads=8, head_dim=128, page_size=16, qo_indptr=b.qo_indptr, causal=True,
                 num_workers=C)
    ws = api.alloc_workspace(p)
    p.upload(ws)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], 32, dtype=torch.float32, device="cuda")
    sm = 1.0 / math.sqrt(128)

    def step(s):
        api.run_prefill(p, ws, q, k, v, o=o, lse=lse, sm_scale=sm)

    n = max(3, args.steps // 4)
    ms = time_calls(step, n, 2)
    attn_ms, _, merge_ms, _ = kernel_times(step, 5)
    fl = prefill_flops(b.kv_lens, 32, 128)
    return {"ms": ms, "tflops": fl / (ms * 1e-3) / 1e12, "flops": fl, "attn_kernel_ms": attn_ms,
            "merge_kernel_ms": merge_ms, "num_workers": C, "lens_sum": int(b.kv_lens.sum())}


def cpu_baseline(dec):
    """The fp64 numpy oracle on a bounded sample of the decode batch (first requests until
    ~15 s of CPU work), reported in the same unit (GB/s of algorithmic bytes)."""
    from oracle import attention as A

    b = dec["batch"]
    cores = len(os.sched_getaffinity(0))
    done, nbytes = [], 0
    t0 = time.perf_counter()
    for i in range(b.batch):
        A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, 16,
                          32, 8, 1.0 / math.sqrt(128), requests=[i])
        done.append(i)
        if time.perf_counter() - t0 > 15.0:
            break
    dt = time.perf_counter() - t0
    lens = b.kv_lens[done]
    nbytes = decode_bytes(lens, len(done), 32, 8, 128, int(sum((l + 15) // 16 for l in lens)))
    try:
        import threadpoolctl

        blas = max((x.get("num_threads", 1) for x in threadpoolctl.threadpool_info()), default=1)
    except Exception:
        blas = None
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "blas_threads": blas,
            "sample": f"fp64 numpy oracle on the first {len(done)} of 64 decode requests "
                      f"({int(lens.sum())} KV tokens), {dt:.1f} s wall"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="decode only, no CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this attention path has no multi-GPU part "
              "(every GPU would run the same kernels on its own requests); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    log(f"device: {torch.cuda.get_device_name(0)}  torch {torch.__version__}")
    dec = bench_decode(args)
    log(f"decode: {dec['ms_per_step']*1e3:.1f} us/step, {dec['gbs']:.0f} GB/s; attn kernel "
        f"{dec['attn_kernel_ms']*1e3:.1f} us, merge {dec['merge_kernel_ms']*1e3:.1f} us")
    out = {
        "metric": METRIC,
        "value": round(dec["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, random page permutation)",
        "config": {
            "workload": "batched paged decode bf16: batch 64, KV lengths U[512,8192], page size 16, "
                        "32 query / 8 KV heads, head_dim 128, split-KV + merge",
            "tokens": dec["tokens"], "algorithmic_bytes": dec["bytes"],
            "num_workers": dec["num_workers"], "work_items": dec["num_items"],
            "partial_slots": dec["num_slots"], "plan_host_us": round(dec["plan_host_us"], 1),
            "median_us": round(dec["median_ms"] * 1e3, 2), "min_us": round(dec["min_ms"] * 1e3, 2),
            "p90_us": round(dec["p90_ms"] * 1e3, 2),
            "pct_hbm_peak": round(100 * dec["gbs"] / HBM_PEAK_GBS, 2),
        },
    }
    ach = dec["bytes"] / (dec["attn_kernel_ms"] * 1e-3) / 1e9
    out["roofline"] = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                       "kernel": "attn_decode_bf16_kernel<128,4>",
                       "kernel_avg_us": round(dec["attn_kernel_ms"] * 1e3, 2),
                       "merge_avg_us": round(dec["merge_kernel_ms"] * 1e3, 2)}
    if not args.quick:
        pf = bench_prefill(args)
        log(f"prefill: {pf['ms']*1e3:.1f} us, {pf['tflops']:.1f} TFLOP/s")
        out["prefill"] = {"workload": "ragged causal prefill bf16: batch 16, q_len = kv_len U[256,4096], "
                                      "page size 16, 32/8 heads, head_dim 128",
                          "tflops": round(pf["tflops"], 2), "ms": round(pf["ms"], 4),
                          "pct_bf16_peak": round(100 * pf["tflops"] / BF16_PEAK_TFLOPS, 2),
                          "attn_kernel_ms": round(pf["attn_kernel_ms"], 4),
                          "merge_kernel_ms": round(pf["merge_kernel_ms"], 4),
                          "flops": pf["flops"], "num_workers": pf["num_workers"]}
        out["cpu_baseline"] = cpu_baseline(dec)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
