"""Benchmark of the block-sparse paged attention path on one MI355X.

One step = one bsr_run_decode call on the batch-64 paged decode workload (bf16,
KV lengths U[512, 8192], page size 16, 32 query / 8 KV heads, head_dim 128): one launch
of the attention kernel over the planned split-KV partition, which also folds the split
requests' partial states.  The plan is built once and reused by every step (one plan per generation
step serves all layers).  Inputs are resident in HBM before timing; three copies of
the KV pool are rotated so the last-level cache cannot serve a step from the previous
one.  The same JSON line also reports
  - the ragged causal prefill (batch 16, q_len = kv_len U[256, 4096]) in TFLOP/s,
  - page size 1 (rows scattered over a 2^20-row pool) next to the same contents laid
    out contiguously, for the decode batch and for a batch-8 2048-token causal prefill,
  - the composable shared-prefix decode (16 groups x 4 requests, 2048-token prefix
    per group at 4 queries per block row + private suffixes, merged) and its
    single-level baseline,
  - a three-level cascade, and one prefix shared by a whole batch (batch 64 with a
    32,768-token prefix, batch 16 with 1,024; 128-token suffixes) composed and single-level,
  - the attention variants (soft cap, sliding window, tree masks) and E4M3 KV decode,
  - the roofline of the decode call (timed with HIP events over the timed region, on the stream
    it runs on), next to the streaming-read ceiling of the same pages (libbsr_probe.so, measured
    in the run), and of the prefill kernel, with per-kernel averages and HBM counters from the
    committed rocprofv3 summaries while the kernel sources match,
  - the fp64 CPU oracle timed on the host cores as a baseline, for decode and for prefill.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--only NAME]
                       [--copy-calib]
       python bench.py --profile-commands NAME   (the rocprofv3 runs behind profiles/NAME.*)
       python bench.py --profile-case NAME       (one case's calls only, run under rocprofv3)
       python bench.py --summarize NAME          (profiles/NAME.json and .md from their output)
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
H_QO, H_KV, D = 32, 8, 128
SM = 1.0 / math.sqrt(D)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(kv_lens, B, nnz, elt=2):
    """Algorithmic bytes of one decode call: K and V read once (one KV head serves its g
    query heads), Q read, O and LSE written, page table (indices, indptr, last lengths)."""
    kv = int(np.sum(kv_lens)) * H_KV * D * elt * 2
    qo = 2 * B * H_QO * D * elt
    return kv + qo + B * H_QO * 4 + nnz * 4 + (B + 1) * 4 + B * 4


def prefill_flops(lens):
    """QK^T and PV flops over the unmasked (causal, bottom-right) pairs only."""
    return float(sum(4.0 * D * H_QO * l * (l + 1) / 2 for l in lens))


def time_calls(fn, steps, warmup):
    import torch

    for s in range(warmup):
        fn(s)
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


def make_plan(b, kind, causal=False, affine=False, **variant):
    """affine: plan the batch as a contiguous cache (no page table; its table must be the identity)."""
    from block_sparse_paged_bsr_amd import api

    C = api.query_num_workers(kind, H_QO, H_KV, D)
    if affine:
        assert np.array_equal(b.kv_indices, np.arange(len(b.kv_indices)))
    return api.Plan(b.kv_indptr, None if affine else b.kv_indices, b.last_page_len, num_pages=b.num_pages,
                    num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D, page_size=b.page_size,
                    qo_indptr=b.qo_indptr, causal=causal, num_workers=C, **variant)


def run_case(b, kind, steps, warmup, rotate=1, causal=False, **variant):
    """Plan once, upload, then time steps of run_decode / run_prefill."""
    import torch
    from block_sparse_paged_bsr_amd import api

    q, k, v = b.torch_values("cuda")
    p = make_plan(b, kind, causal, **variant)
    # host planning time of a warm call (the first one also pays for the worker-count query)
    plan_us = float("inf")
    for _ in range(3):
        t0 = time.perf_counter()
        make_plan(b, kind, causal, **variant)
        plan_us = min(plan_us, (time.perf_counter() - t0) * 1e6)
    ws = api.alloc_workspace(p)
    p.upload(ws)
    # the plan's metadata copy on its own (a second upload: the first one also sets up the
    # pinned staging), timed with events on the stream it runs on
    torch.cuda.synchronize()
    u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    u0.record()
    p.upload(ws)
    u1.record()
    torch.cuda.synchronize()
    upload_us = u0.elapsed_time(u1) * 1e3
    pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(rotate - 1)]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], H_QO, dtype=torch.float32, device="cuda")
    fn = api.run_decode if kind == "decode" else api.run_prefill

    def step(s):
        kk, vv = pools[s % len(pools)]
        fn(p, ws, q, kk, vv, o=o, lse=lse, sm_scale=SM)

    ms = time_calls(step, steps, warmup)
    e = p.export()
    res = {"ms": ms, "plan_us": plan_us, "upload_us": upload_us, "meta_bytes": int(p.workspace_bytes()),
           "num_workers": e["num_workers"],
           "items": int(e["items"].shape[0]), "slots": e["num_slots"], "step": step,
           "out": (o, lse), "pools": pools}
    return res


def read_ceiling(pools, pages, steps, warmup, per_cu=(2, 4, 8, 16)):
    """Streaming-read ceiling of the decode access shape on this device: libbsr_probe.so reads the
    pages the call reads (every listed page of K and of V, in page-table order, whole pages, the
    same rotated pools) and does nothing else with them.  Best of a few grid sizes, timed like the
    call (events around back-to-back launches on the stream they run on)."""
    import ctypes
    import torch
    from block_sparse_paged_bsr_amd import _lib

    L = _lib.probe()
    k0 = pools[0][0]
    page_bytes = k0[0].numel() * k0.element_size()
    pg = torch.from_numpy(np.ascontiguousarray(pages, dtype=np.int32)).to("cuda")
    assert int(pg.min()) >= 0 and int(pg.max()) < k0.shape[0]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    best = None
    for n in per_cu:
        grid = cus * n
        sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")

        def step(s, grid=grid, sink=sink):
            kk, vv = pools[s % len(pools)]
            rc = L.bsr_probe_read_pages(ctypes.c_void_p(kk.data_ptr()), ctypes.c_void_p(vv.data_ptr()),
                                        ctypes.c_void_p(pg.data_ptr()), int(pg.numel()), page_bytes, grid,
                                        0x9E3779B9, ctypes.c_void_p(sink.data_ptr()),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            assert rc == 0, rc

        ms = time_calls(step, steps, warmup)
        nbytes = 2 * int(pg.numel()) * page_bytes
        gbs = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": round(gbs, 1), "us": round(ms * 1e3, 2), "grid": grid, "bytes": nbytes}
    best["kernel"] = "bsr_probe_read_pages (libbsr_probe.so)"
    return best


ISA_MIX_MODES = ["MFMA", "MFMA + 6 FMA", "MFMA + 8 FMA", "MFMA + 3 EXP", "MFMA + 4 EXP", "8 FMA", "8 EXP",
                 "MFMA + 2 FMA + 2 EXP"]  # the slots of bsr_probe_issue_mix (include/bsr_probe.h)


def isa_rates(out_md=None, iters=4096):
    """Execution rates of the device behind the kernels' design (libbsr_probe.so execution-rate
    probes): cycles per slot of the one-wave instruction mixes, LDS read rates of the prefill
    kernel's operand patterns, and the L2-to-LDS copy rate of a CU.  Returns a dict; with out_md,
    also writes it as a markdown table with the command that produced it."""
    import ctypes
    import torch
    from block_sparse_paged_bsr_amd import _lib

    L = _lib.probe()
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)  # noqa: E731
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    cyc = torch.zeros(4 * 1024, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    res = {"issue_mix_cycles_per_slot": {}, "lds_read": {}, "l2_to_lds": {}}
    for mode, name in enumerate(ISA_MIX_MODES):
        for n in (16, iters):  # the first launch warms the code up
            assert L.bsr_probe_issue_mix(mode, n, vp(cyc), vp(sink), st()) == 0
        torch.cuda.synchronize()
        c = cyc[:2].cpu().tolist()
        res["issue_mix_cycles_per_slot"][name] = round(c[0] / (8.0 * iters), 2)
        res["clock_ghz"] = round(c[0] / (c[1] * 10.0), 3)
    for pattern, (pname, per, nbytes) in enumerate((("ds_read_b128 (K pattern)", 8, 1024),
                                                    ("ds_read_b64_tr_b16 (V pattern)", 16, 512))):
        for waves in (1, 2, 4):
            for n in (8, iters // 4):
                assert L.bsr_probe_lds_read(pattern, waves, n, vp(cyc), vp(sink), st()) == 0
            torch.cuda.synchronize()
            mx = max(cyc[:waves].cpu().tolist())
            n = iters // 4
            res["lds_read"][f"{pname}, {waves} wave(s)"] = {
                "cycles_per_instruction": round(mx / (n * per), 2),
                "bytes_per_cycle_per_cu": round(n * per * nbytes * waves / mx, 1)}
    src = torch.ones(1 << 16, dtype=torch.int32, device="cuda")  # 256 KB, L2-resident
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for waves, blocks in ((1, 1), (4, 1), (4, cus), (4, 2 * cus)):
        for n in (8, iters // 4):
            assert L.bsr_probe_l2_to_lds(vp(src), waves, blocks, n, vp(cyc), vp(sink), st()) == 0
        torch.cuda.synchronize()
        c = cyc[:4 * blocks].view(blocks, 4)[:, :waves]
        mx = int(c.max())
        n = iters // 4
        per_cu = max(1, blocks // cus)  # workgroups sharing a CU
        res["l2_to_lds"][f"{waves} wave(s) x {blocks} workgroup(s)"] = {
            "cycles_per_8kb": round(mx / n, 1),
            "bytes_per_cycle_per_cu": round(8192.0 * n * waves * per_cu / mx, 1)}
    if out_md:
        cmd = "python3 bench.py --isa-rates " + os.path.basename(out_md)
        lines = ["# Execution rates of the device (libbsr_probe.so execution-rate probes)", "",
                 f"Command: `{cmd}` (shader-clock cycles from s_memtime; clock {res['clock_ghz']} GHz "
                 "from the same loop's real-time counter).", "",
                 "One wave, cycles per slot (a slot = at most one `v_mfma_f32_32x32x16_bf16` and the vector "
                 "instructions listed; each vector instruction reads a value written two slots earlier):", "",
                 "| Slot | Cycles |", "|---|---|"]
        lines += [f"| {k} | {v} |" for k, v in res["issue_mix_cycles_per_slot"].items()]
        lines += ["", "LDS reads of the 128-row prefill kernel's operand patterns (one workgroup):", "",
                  "| Pattern | Cycles per instruction per wave | Bytes per cycle per CU |", "|---|---|---|"]
        lines += [f"| {k} | {v['cycles_per_instruction']} | {v['bytes_per_cycle_per_cu']} |"
                  for k, v in res["lds_read"].items()]
        lines += ["", "L2 to LDS (eight 1 KB `global_load_lds_dwordx4` per wave, then a wait; source L2-resident):", "",
                  "| Waves x workgroups | Cycles per 8 KB per wave | Bytes per cycle per CU |", "|---|---|---|"]
        lines += [f"| {k} | {v['cycles_per_8kb']} | {v['bytes_per_cycle_per_cu']} |" for k, v in res["l2_to_lds"].items()]
        with open(out_md, "w") as f:
            f.write("\n".join(lines) + "\n")
    return res


def graph_replay_ms(step, steps, warmup, variants=3):
    """Per-step time when each step is a captured HIP graph replayed (one graph per KV pool
    of the rotation): the plan-once, replay-per-step loop of a serving engine."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(variants):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for i in range(variants):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    return time_calls(lambda s: graphs[s % variants].replay(), steps, warmup)


def bench_decode(args):
    import workloads as inputs

    b = inputs.batched_decode_bf16(seed=0, poison=False)
    r = run_case(b, "decode", args.steps, args.warmup, rotate=3)
    med, mn, p90 = per_call_ms(r["step"], 50 if not args.quick else 10)
    graph_ms = graph_replay_ms(r["step"], args.steps, args.warmup)
    nbytes = decode_bytes(b.kv_lens, b.batch, len(b.kv_indices))
    ceiling = read_ceiling(r.pop("pools"), b.kv_indices, args.steps, args.warmup)
    r.update({"gbs": nbytes / (r["ms"] * 1e-3) / 1e9, "bytes": nbytes, "median_ms": med, "min_ms": mn,
              "p90_ms": p90, "graph_ms": graph_ms, "read_ceiling": ceiling,
              "tokens": int(b.kv_lens.sum()), "batch": b})
    return r


def bench_prefill(args):
    import workloads as inputs

    b = inputs.ragged_prefill_bf16(seed=0, poison=False)
    # ~1 ms per call: enough warm-up calls for the clocks to settle, then a few tens timed
    r = run_case(b, "prefill", max(10, args.steps // 2), 10, causal=True)
    fl = prefill_flops(b.kv_lens)
    return {"ms": r["ms"], "tflops": fl / (r["ms"] * 1e-3) / 1e12, "flops": fl, "num_workers": r["num_workers"],
            "slots": r["slots"], "batch": b}


def windowed_prefill_flops(lens, w):
    """Flops over the visible pairs of causal prefill with a window of w keys to the left:
    query position p (0-based, q_len = kv_len) sees min(p + 1, w + 1) keys."""
    tot = 0.0
    for l in lens:
        l = int(l)
        full = min(l, w + 1)  # positions 0 .. full-1 see p + 1 keys
        tot += full * (full + 1) / 2 + (l - full) * (w + 1)
    return 4.0 * D * H_QO * tot


def bench_variants(args):
    """The attention variants on the headline workloads: logits soft cap 50 and a 4096-key
    sliding window on batch-64 decode; 16 speculative draft tokens per decode request under a
    tree mask (custom mask) and under the causal mask; soft cap 50, a 1024-key window, and
    both, on the ragged causal prefill.  Rates count only the visible KV (window) or pairs."""
    import workloads as inputs

    out = {}
    b = inputs.batched_decode_bf16(seed=0, poison=False)
    nnz = len(b.kv_indices)
    for name, var, lens in (("decode_soft_cap50", dict(logits_soft_cap=50.0), b.kv_lens),
                            ("decode_window4096", dict(window_left=4095), np.minimum(b.kv_lens, 4096))):
        r = run_case(b, "decode", args.steps, args.warmup, rotate=3, **var)
        nbytes = decode_bytes(lens, b.batch, nnz if "window" not in name else int(np.sum((lens + 15) // 16)))
        out[name] = {"us": round(r["ms"] * 1e3, 2), "gbs": round(nbytes / (r["ms"] * 1e-3) / 1e9, 1),
                     "bytes": nbytes}
        del r
    # speculative decoding: 16 draft tokens per request of the batch-64 decode workload, each
    # seeing the prompt and its ancestors in a random tree (custom mask) vs the causal mask
    import torch
    from block_sparse_paged_bsr_amd import api

    rng = np.random.default_rng(0)
    T = 16
    prompt = inputs.decode_lengths(0)
    sb = inputs.make_paged_batch(0, prompt + T, np.full(len(prompt), T), page_size=16, num_qo_heads=H_QO,
                                 num_kv_heads=H_KV, head_dim=D, poison=False)
    masks = []
    for L in prompt:
        m = np.zeros((T, int(L) + T), dtype=bool)
        m[:, :L] = True
        par = [-1] + [int(rng.integers(-1, t)) for t in range(1, T)]
        for t in range(T):
            a_ = t
            while a_ >= 0:
                m[t, L + a_] = True
                a_ = par[a_]
        masks.append(m)
    bits = torch.from_numpy(api.pack_custom_mask(masks)).to("cuda")
    q, k, v = sb.torch_values("cuda")
    spec_bytes = int(sb.kv_lens.sum()) * H_KV * D * 2 * 2
    for name, causal, use_mask in (("spec_tree_mask16", False, True), ("spec_causal16", True, False)):
        p = make_plan(sb, "prefill", causal)
        ws = api.alloc_workspace(p)
        p.upload(ws)
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[0], H_QO, dtype=torch.float32, device="cuda")
        if use_mask:
            step = lambda s_: api.run_prefill_masked(p, ws, q, k, v, bits, o=o, lse=lse, sm_scale=SM)
        else:
            step = lambda s_: api.run_prefill(p, ws, q, k, v, o=o, lse=lse, sm_scale=SM)
        ms = time_calls(step, args.steps, args.warmup)
        out[name] = {"us": round(ms * 1e3, 2), "kv_gbs": round(spec_bytes / (ms * 1e-3) / 1e9, 1),
                     "tile_q": int(p.export()["tile_q"])}
    del q, k, v, bits
    torch.cuda.empty_cache()
    pb = inputs.ragged_prefill_bf16(seed=0, poison=False)
    for name, var, fl in (("prefill_soft_cap50", dict(logits_soft_cap=50.0), prefill_flops(pb.kv_lens)),
                          ("prefill_window1024", dict(window_left=1024), windowed_prefill_flops(pb.kv_lens, 1024)),
                          ("prefill_window1024_soft_cap50", dict(window_left=1024, logits_soft_cap=50.0),
                           windowed_prefill_flops(pb.kv_lens, 1024))):
        r = run_case(pb, "prefill", max(10, args.steps // 2), 10, causal=True, **var)
        out[name] = {"ms": round(r["ms"], 4), "tflops": round(fl / (r["ms"] * 1e-3) / 1e12, 1), "flops": fl}
        del r
    return out


def bench_e4m3(args, num_workers=None):
    """Batch-64 paged decode with K and V stored as E4M3 bytes (per-tensor scales): the same
    requests and page tables as the bf16 headline, half the KV bytes."""
    import torch
    from block_sparse_paged_bsr_amd import api
    import workloads as inputs

    b = inputs.batched_decode_bf16(seed=0, poison=False)
    e = inputs.to_e4m3(b)
    q, k, v = e.torch_values("cuda")
    C = num_workers or api.query_num_workers("decode", H_QO, H_KV, D)
    p = api.Plan(b.kv_indptr, b.kv_indices, b.last_page_len, num_pages=b.num_pages, num_qo_heads=H_QO,
                 num_kv_heads=H_KV, head_dim=D, page_size=b.page_size, num_workers=C)
    ws = api.alloc_workspace(p)
    p.upload(ws)
    pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(2)]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], H_QO, dtype=torch.float32, device="cuda")

    def step(s):
        kk, vv = pools[s % len(pools)]
        api.run_decode_e4m3(p, ws, q, kk, vv, e.k_scale, e.v_scale, o=o, lse=lse, sm_scale=SM)

    ms = time_calls(step, args.steps, args.warmup)
    nbytes = decode_bytes(b.kv_lens, b.batch, len(b.kv_indices), elt=1) + 2 * b.batch * H_QO * D  # Q/O stay bf16
    return {"us": round(ms * 1e3, 2), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "bytes": nbytes, "num_workers": C,
            "k_scale": e.k_scale, "v_scale": e.v_scale}


def bench_vector_sparse(args):
    """Page size 1 over a 2^20-row pool vs the same contents contiguous: through the identity
    page table (same loader, row locality only) and, for decode, planned as a contiguous cache
    (page ids computed: the cost of indexed addressing)."""
    import workloads as inputs

    out = {}
    lens = inputs.decode_lengths(0)
    a, c = inputs.vector_sparse_pair(0, lens, pool_rows=1 << 20)
    nbytes = decode_bytes(lens, len(lens), len(a.kv_indices))
    ra = run_case(a, "decode", args.steps, args.warmup)
    rc = run_case(c, "decode", args.steps, args.warmup)
    # the contiguous twin once more, planned without a page table: page ids computed, not loaded
    rf = run_case(c, "decode", args.steps, args.warmup, affine=True)
    out["decode"] = {"paged_us": round(ra["ms"] * 1e3, 2), "contiguous_us": round(rc["ms"] * 1e3, 2),
                     "contiguous_affine_us": round(rf["ms"] * 1e3, 2),
                     "paged_gbs": round(nbytes / (ra["ms"] * 1e-3) / 1e9, 1),
                     "contiguous_gbs": round(nbytes / (rc["ms"] * 1e-3) / 1e9, 1),
                     "contiguous_affine_gbs": round(nbytes / (rf["ms"] * 1e-3) / 1e9, 1),
                     "paged_over_contiguous_time": round(ra["ms"] / rc["ms"], 4),
                     "paged_over_affine_time": round(ra["ms"] / rf["ms"], 4)}
    del a, c, ra, rc, rf
    plens = [2048] * 8
    a, c = inputs.vector_sparse_pair(1, plens, plens, pool_rows=1 << 20, causal=True)
    fl = prefill_flops(plens)
    ra = run_case(a, "prefill", max(5, args.steps // 5), 2, causal=True)
    rc = run_case(c, "prefill", max(5, args.steps // 5), 2, causal=True)
    out["prefill"] = {"paged_us": round(ra["ms"] * 1e3, 2), "contiguous_us": round(rc["ms"] * 1e3, 2),
                      "paged_tflops": round(fl / (ra["ms"] * 1e-3) / 1e12, 1),
                      "contiguous_tflops": round(fl / (rc["ms"] * 1e-3) / 1e12, 1),
                      "paged_over_contiguous_time": round(ra["ms"] / rc["ms"], 4)}
    return out


def bench_composable(args):
    """Two BSR views (shared prefix at 4 queries per block row, private suffixes) merged,
    vs the single-level view (each request reads prefix ++ suffix itself)."""
    import torch
    from block_sparse_paged_bsr_amd import api
    import workloads as inputs

    b = inputs.shared_prefix_decode(seed=0, poison=False)
    q, k, v = b.torch_values("cuda")
    # (the prefix level's block rows are 16-row tiles of 4 queries: the decode kernel serves them)
    C2 = api.query_num_workers("decode", H_QO, H_KV, D)
    p1 = api.Plan(b.l1_kv_indptr, b.l1_kv_indices, b.l1_last_page_len, num_pages=b.num_pages,
                  num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D, page_size=b.page_size,
                  qo_indptr=b.l1_qo_indptr, causal=False, num_workers=C2)
    p2 = api.Plan(b.l2_kv_indptr, b.l2_kv_indices, b.l2_last_page_len, num_pages=b.num_pages,
                  num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D, page_size=b.page_size, num_workers=C2)
    pf = api.Plan(b.full_kv_indptr, b.full_kv_indices, b.full_last_page_len, num_pages=b.num_pages,
                  num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D, page_size=b.page_size, num_workers=C2)
    w1, w2, wf = api.alloc_workspace(p1), api.alloc_workspace(p2), api.alloc_workspace(pf)
    p1.upload(w1)
    p2.upload(w2)
    pf.upload(wf)
    R = q.shape[0]
    o1, o2, o = (torch.empty_like(q) for _ in range(3))
    l1, l2, l = (torch.empty(R, H_QO, dtype=torch.float32, device="cuda") for _ in range(3))

    # the pool (~280 MB) is near the last-level cache size: rotate three copies
    pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(2)]

    def composed(s):
        kk, vv = pools[s % 3]
        api.run_prefill(p1, w1, q, kk, vv, o=o1, lse=l1, sm_scale=SM)
        api.run_decode(p2, w2, q, kk, vv, o=o2, lse=l2, sm_scale=SM)
        api.merge_state(o1, l1, o2, l2, o_out=o, lse_out=l)

    # the same two views as one composable plan: one attention launch over both views' block
    # rows (decode kernel, 16-row tiles), one merge launch folding each query's states
    cp = api.ComposablePlan([dict(kv_indptr=b.l1_kv_indptr, kv_indices=b.l1_kv_indices,
                                  last_page_len=b.l1_last_page_len, qo_indptr=b.l1_qo_indptr),
                             dict(kv_indptr=b.l2_kv_indptr, kv_indices=b.l2_kv_indices,
                                  last_page_len=b.l2_last_page_len)],
                            num_pages=b.num_pages, num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D,
                            page_size=b.page_size, num_workers=C2)
    wc = api.alloc_workspace(cp)
    cp.upload(wc)

    def one_plan(s):
        kk, vv = pools[s % 3]
        api.run_prefill(cp, wc, q, kk, vv, o=o, lse=l, sm_scale=SM)

    def single(s):
        kk, vv = pools[s % 3]
        api.run_decode(pf, wf, q, kk, vv, o=o, lse=l, sm_scale=SM)

    ms_p = time_calls(one_plan, args.steps, args.warmup)
    ms_c = time_calls(composed, args.steps, args.warmup)
    ms_s = time_calls(single, args.steps, args.warmup)
    ms_pg = graph_replay_ms(one_plan, args.steps, args.warmup)
    ms_cg = graph_replay_ms(composed, args.steps, args.warmup)
    ms_sg = graph_replay_ms(single, args.steps, args.warmup)
    per = H_KV * D * 2 * 2
    qol = 2 * R * H_QO * D * 2 + R * H_QO * 4
    comp_bytes = b.groups * b.prefix_len * per + int(b.suffix_lens.sum()) * per + qol
    single_bytes = int((b.prefix_len + b.suffix_lens).sum()) * per + qol
    ce = cp.export()
    return {"composable_us": round(ms_p * 1e3, 2), "single_level_us": round(ms_s * 1e3, 2),
            "speedup": round(ms_s / ms_p, 3), "composable_bytes": comp_bytes, "single_level_bytes": single_bytes,
            "composable_gbs_counted": round(comp_bytes / (ms_p * 1e-3) / 1e9, 1),
            "pct_hbm_peak_counted": round(100 * comp_bytes / (ms_p * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
            "single_level_gbs": round(single_bytes / (ms_s * 1e-3) / 1e9, 1),
            "traffic_ratio_eq15": round(single_bytes / comp_bytes, 3),
            "composable_plan": {"launches": 2, "workers": C2, "chunks": int(ce["items"].shape[0]),
                                "partial_slots": ce["num_slots"], "graph_us": round(ms_pg * 1e3, 2)},
            "two_plans_and_merge_state_us": round(ms_c * 1e3, 2),
            "two_plans_graph_us": round(ms_cg * 1e3, 2), "single_level_graph_us": round(ms_sg * 1e3, 2),
            "graph_speedup": round(ms_sg / ms_pg, 3)}


def cpu_baseline(dec):
    """The fp64 numpy oracle, as it stands, on the decode batch (whole requests until ~12 s
    of CPU work), reported in the same unit (GB/s of algorithmic bytes)."""
    from oracle import attention as A

    b = dec["batch"]
    cores = len(os.sched_getaffinity(0))
    done = []
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < 12.0:
        for i in range(b.batch):
            A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len,
                              16, H_QO, H_KV, SM, requests=[i])
            done.append(i)
            if time.perf_counter() - t0 > 12.0:
                break
        reps += 1
    dt = time.perf_counter() - t0
    lens = b.kv_lens[done]
    nbytes = decode_bytes(lens, len(done), int(sum((l + 15) // 16 for l in lens)))
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "blas_threads": _blas_threads(),
            "sample": f"fp64 numpy oracle, {len(done)} request evaluations of the batch-64 decode "
                      f"({int(lens.sum())} KV tokens, {reps} pass(es)), {dt:.1f} s wall"}


def cpu_baseline_prefill(pf):
    """The fp64 numpy oracle, as it stands, on whole requests of the ragged causal prefill
    (shortest first, until ~10 s of CPU work), in the GPU metric's unit: algorithmic TFLOP/s
    (QK^T and PV over the unmasked pairs; the oracle itself multiplies the full l x l products)."""
    from oracle import attention as A

    b = pf["batch"]
    cores = len(os.sched_getaffinity(0))
    done = []
    t0 = time.perf_counter()
    for i in np.argsort(b.kv_lens, kind="stable"):
        A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, 16, H_QO, H_KV, SM,
                          qo_indptr=b.qo_indptr, causal=True, requests=[int(i)])
        done.append(int(i))
        if time.perf_counter() - t0 > 10.0:
            break
    dt = time.perf_counter() - t0
    fl = prefill_flops(b.kv_lens[done])
    return {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "blas_threads": _blas_threads(),
            "sample": f"fp64 numpy oracle on {len(done)} whole requests of the ragged causal prefill "
                      f"(lengths {sorted(int(b.kv_lens[i]) for i in done)}), {dt:.1f} s wall"}


def _blas_threads():
    try:
        import threadpoolctl

        return max((x.get("num_threads", 1) for x in threadpoolctl.threadpool_info()), default=1)
    except Exception:
        return None


def profile_record(name):
    """A committed rocprofv3 summary (profiles/<name>.json: kernel-trace averages, HBM counters),
    used only while every kernel source it was taken on is unchanged (SHA-256), else None."""
    import hashlib

    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", name + ".json")))
        for src, sha in rec["sources"].items():
            if hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != sha:
                return None
    except (OSError, ValueError, KeyError):
        return None
    return rec


def copy_calibration():
    """A plain 512 MiB device copy (torch), so counter runs can scale FETCH_SIZE/WRITE_SIZE."""
    import torch

    n = 512 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 x {n} bytes")


# ---- rocprofv3 summaries (profiles/<name>.json, .md) ----
# Each case runs one call of the path, warm-up and timed steps only, so that the kernel-trace
# averages and the counters of its kernels belong to that call alone.
SRC = "block_sparse_paged_bsr_amd/csrc/kernels/"
PROFILE_CASES = {
    "decode_batch64": {
        "workload": "batched paged decode bf16: batch 64, KV lengths U[512,8192], page size 16, 32 query / "
                    "8 KV heads, head_dim 128 (seed 0)",
        "kernels": {"attn_decode_bf16_kernel": "attention, split requests folded in the kernel (the whole call)",
                    "read_pages_kernel": "HBM read probe: the same K/V pages, page-table order, nothing else"},
        "call": ["attn_decode_bf16_kernel"],
        "sources": [SRC + "attn_decode_bf16.hip", SRC + "common.h", "block_sparse_paged_bsr_amd/csrc/hbm_probe.hip"],
        "unit": "bytes"},
    "prefill_ragged": {
        "workload": "ragged causal prefill bf16: batch 16, q_len = kv_len U[256,4096], page size 16, 32 query / "
                    "8 KV heads, head_dim 128 (seed 0)",
        "kernels": {"attn_prefill128_bf16_kernel": "attention, 128-row query tiles"},
        "call": ["attn_prefill128_bf16_kernel"],
        "sources": [SRC + "attn_prefill_bf16.hip", SRC + "common.h"],
        "unit": "flops", "sq": True, "traffic": True},
    "composable_shared_prefix": {
        "workload": "composable shared-prefix decode bf16: 16 groups x 4 requests, 2048-token prefix per group, "
                    "private suffixes U[128,1024], page size 16, 32/8 heads, head_dim 128 (seed 0), one plan",
        "kernels": {"attn_decode_bf16_kernel": "attention over both levels' 16-row tiles",
                    "merge_partials_kernel": "fold of each query's states over chunks and levels"},
        "call": ["attn_decode_bf16_kernel", "merge_partials_kernel"],
        "sources": [SRC + "attn_decode_bf16.hip", SRC + "merge.hip", SRC + "common.h",
                    "block_sparse_paged_bsr_amd/csrc/compose.cpp"],
        "unit": "bytes"},
    "decode_page1": {
        "workload": "batched paged decode bf16 at page size 1: the batch-64 decode's tokens scattered one per "
                    "page over a 2^20-row pool (seed 0)",
        "kernels": {"attn_decode_bf16_kernel": "attention, split requests folded in the kernel (the whole call)"},
        "call": ["attn_decode_bf16_kernel"],
        "sources": [SRC + "attn_decode_bf16.hip", SRC + "common.h"],
        "unit": "bytes"},
}
SQ_COUNTERS = ("GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS "
               "SQ_WAVE_CYCLES SQ_WAIT_INST_ANY")
PROFILE_STEPS = "--steps 20 --warmup 5"
PROFILE_RAW = "rocprof_out"  # rocprofv3 output of the profile runs, relative to the repository root


def profile_commands(name):
    """The rocprofv3 runs behind profiles/<name>.json, from the repository root: a kernel trace,
    then FETCH_SIZE and WRITE_SIZE passes (each with the copy calibration) for the HBM-bound
    cases, SQ counters for prefill."""
    case = PROFILE_CASES[name]
    run = f"python3 bench.py --profile-case {name} {PROFILE_STEPS}"
    d = f"{PROFILE_RAW}/{name}"
    cmds = [f"timeout -s KILL 300 rocprofv3 --kernel-trace --stats --output-format csv -d {d}_trace -o run -- {run} "
            f"--profile-out {d}_event.json"]
    if case["unit"] == "bytes" or case.get("traffic"):
        cmds += [f"timeout -s KILL 300 rocprofv3 --pmc FETCH_SIZE --output-format csv -d {d}_fetch -o run -- {run} "
                 "--copy-calib",
                 f"timeout -s KILL 300 rocprofv3 --pmc WRITE_SIZE --output-format csv -d {d}_write -o run -- {run} "
                 "--copy-calib"]
    if case.get("sq"):
        cmds.append(f"timeout -s KILL 300 rocprofv3 --pmc {SQ_COUNTERS} --output-format csv -d {d}_sq -o run -- {run}")
    return cmds


def profile_case_batch(name):
    import workloads as inputs

    if name == "decode_batch64":
        return inputs.batched_decode_bf16(seed=0, poison=False)
    if name == "prefill_ragged":
        return inputs.ragged_prefill_bf16(seed=0, poison=False)
    if name == "composable_shared_prefix":
        return inputs.shared_prefix_decode(seed=0, poison=False)
    if name == "decode_page1":
        return inputs.vector_sparse_pair(0, inputs.decode_lengths(0), pool_rows=1 << 20)[0]
    raise KeyError(name)


def profile_algorithmic(name, b):
    """Algorithmic bytes (or flops) of one call of the case."""
    if name in ("decode_batch64", "decode_page1"):
        return decode_bytes(b.kv_lens, b.batch, len(b.kv_indices))
    if name == "prefill_ragged":
        return prefill_flops(b.kv_lens)
    per = H_KV * D * 2 * 2  # K and V of one token, all KV heads
    R = int(b.q_f32.shape[0])  # one query per request
    return b.groups * b.prefix_len * per + int(b.suffix_lens.sum()) * per + 2 * R * H_QO * D * 2 + R * H_QO * 4


def run_profile_case(name, args):
    """Warm-up and timed calls of one case and nothing else (plus the read probe for decode)."""
    import torch
    from block_sparse_paged_bsr_amd import api

    b = profile_case_batch(name)
    if name == "composable_shared_prefix":
        q, k, v = b.torch_values("cuda")
        cp = api.ComposablePlan([dict(kv_indptr=b.l1_kv_indptr, kv_indices=b.l1_kv_indices,
                                      last_page_len=b.l1_last_page_len, qo_indptr=b.l1_qo_indptr),
                                 dict(kv_indptr=b.l2_kv_indptr, kv_indices=b.l2_kv_indices,
                                      last_page_len=b.l2_last_page_len)],
                                num_pages=b.num_pages, num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D,
                                page_size=b.page_size, num_workers=api.query_num_workers("decode", H_QO, H_KV, D))
        wc = api.alloc_workspace(cp)
        cp.upload(wc)
        o, l = torch.empty_like(q), torch.empty(q.shape[0], H_QO, dtype=torch.float32, device="cuda")
        pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(2)]

        def step(s):
            kk, vv = pools[s % 3]
            api.run_prefill(cp, wc, q, kk, vv, o=o, lse=l, sm_scale=SM)

        ms = time_calls(step, args.steps, args.warmup)
    elif name == "prefill_ragged":
        ms = run_case(b, "prefill", args.steps, args.warmup, causal=True)["ms"]
    else:
        r = run_case(b, "decode", args.steps, args.warmup, rotate=3 if name == "decode_batch64" else 1)
        ms = r["ms"]
        if name == "decode_batch64":
            log(f"read probe: {read_ceiling(r['pools'], b.kv_indices, args.steps, args.warmup, per_cu=(8,))}")
    log(f"{name}: {ms * 1e3:.2f} us per call")
    # the event-timed call average of this run, next to the trace (the summary compares the two)
    if args.profile_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.profile_out)), exist_ok=True)
        with open(args.profile_out, "w") as f:
            json.dump({"event_timed_us_per_call": round(ms * 1e3, 2), "steps": args.steps, "warmup": args.warmup}, f)


def summarize_profile(name, raw_dir=None, out_dir=None):
    """profiles/<name>.json and .md from the rocprofv3 output of profile_commands(name) (raw_dir
    and out_dir default to rocprof_out/ and profiles/ under the repository root)."""
    import csv
    import hashlib

    case = PROFILE_CASES[name]
    d = os.path.join(raw_dir or os.path.join(ROOT, PROFILE_RAW), name)
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    rows = list(csv.DictReader(open(os.path.join(d + "_trace", "run_kernel_stats.csv"))))
    disp = list(csv.DictReader(open(os.path.join(d + "_trace", "run_kernel_trace.csv"))))
    warm = int(PROFILE_STEPS.split("--warmup ")[1].split()[0])
    kav, kall = {}, {}
    md_rows = []
    for key, what in case["kernels"].items():
        hit = [r for r in rows if key in r["Name"]]
        assert len(hit) == 1, (key, [r["Name"] for r in hit])
        r = hit[0]
        # the timed calls only: the dispatches after the warm-up ones, in dispatch order
        durs = [(int(x["Dispatch_Id"]), (int(x["End_Timestamp"]) - int(x["Start_Timestamp"])) / 1e3)
                for x in disp if key in x["Kernel_Name"]]
        durs = [u for _, u in sorted(durs)][warm:]
        kav[key] = round(sum(durs) / len(durs), 2)
        kall[key] = round(float(r["AverageNs"]) / 1e3, 2)
        md_rows.append(f"| `{r['Name'].replace('void ', '').replace('(bsr::RunArgs)', '')}` | {what} | {r['Calls']} | "
                       f"{float(r['AverageNs']) / 1e3:,.2f} | {kav[key]:,.2f} | {float(r['MinNs']) / 1e3:,.2f} | "
                       f"{float(r['MaxNs']) / 1e3:,.2f} |")

    def counters(tag, counter):
        rs = [r for r in csv.DictReader(open(os.path.join(d + "_" + tag, "run_counter_collection.csv")))
              if r["Counter_Name"] == counter]
        per = {}
        for r in rs:
            per.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], 0.0])[1] += float(r["Counter_Value"])
        disp = sorted(per.items())
        calib = [v for _, (n, v) in disp if "copyBuffer" in n][:3]
        assert len(calib) == 3, "copy calibration dispatches missing"
        scale = 524288.0 / (sum(calib) / 3)
        out = {}
        for key in case["kernels"]:
            vals = [v for _, (n, v) in disp if key in n]
            out[key] = (sum(vals) / len(vals), len(vals))
        return scale, out

    rec = {"name": name, "workload": case["workload"], "commands": profile_commands(name),
           "sources": {p: hashlib.sha256(open(os.path.join(ROOT, p), "rb").read()).hexdigest()
                       for p in case["sources"]},
           "kernel_avg_us": kav, "kernel_avg_us_all_dispatches": kall}
    ev = os.path.join(d + "_event.json")
    if os.path.exists(ev):
        rec["event_timed_us_per_call"] = json.load(open(ev))["event_timed_us_per_call"]
    alg = profile_algorithmic(name, profile_case_batch(name))
    rec["algorithmic_" + case["unit"] + "_per_call"] = alg
    call_us = sum(kav[k] for k in case["call"])
    rec["call_kernels_us"] = round(call_us, 2)
    md = [f"# {name}: rocprofv3 summary", "", f"Workload: {case['workload']}.", "",
          "Commands (from the repository root; library built in-tree; each pass in its own run):", ""]
    md += ["    " + c for c in rec["commands"]]
    md += ["", f"Kernel trace (`run_kernel_stats.csv` over all dispatches; `run_kernel_trace.csv` for the "
           f"timed calls, i.e. the dispatches after the {warm} warm-up calls):", "",
           "| Kernel | Role | Dispatches | Average, all (us) | Average, timed calls (us) | Min (us) | Max (us) |",
           "|---|---|---|---|---|---|---|"]
    md += md_rows
    if "event_timed_us_per_call" in rec:
        md += ["", f"The same traced run timed its calls with HIP events on their stream: "
               f"{rec['event_timed_us_per_call']:.2f} us per call (the kernels of one call: "
               f"{sum(kav[k] for k in case['call']):.2f} us in the trace).  Under the tracer every dispatch "
               "runs somewhat slower than in an untraced run of bench.py."]
    if case["unit"] == "bytes" or case.get("traffic"):
        fs, fetch = counters("fetch", "FETCH_SIZE")
        ws, write = counters("write", "WRITE_SIZE")
        traffic = {k: int(round((fetch[k][0] * fs + write[k][0] * ws) * 1024)) for k in case["kernels"]}
        rec.update({"fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
                    "fetch_kib_per_dispatch": {k: round(fetch[k][0], 1) for k in case["kernels"]},
                    "write_kib_per_dispatch": {k: round(write[k][0], 1) for k in case["kernels"]},
                    "traffic_bytes_per_dispatch": traffic,
                    "traffic_bytes_per_call": sum(traffic[k] for k in case["call"])})
        if case["unit"] == "bytes":
            rec["traffic_over_algorithmic"] = round(rec["traffic_bytes_per_call"] / alg, 4)
            rec["call_kernels_gbs"] = round(alg / (call_us * 1e-6) / 1e9, 1)
        else:
            rec["hbm_gbs"] = round(rec["traffic_bytes_per_call"] / (call_us * 1e-6) / 1e9, 1)
        md += ["", "HBM counters per dispatch (FETCH_SIZE and WRITE_SIZE passes), scaled by what the same counters "
               "read for the three 512 MiB device copies of `--copy-calib` (524,288 KiB read and written each): "
               f"FETCH_SIZE x {fs:.4f}, WRITE_SIZE x {ws:.4f}.", "",
               "| Kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (scaled) |", "|---|---|---|---|"]
        for k in case["kernels"]:
            md.append(f"| `{k}` | {fetch[k][0]:,.1f} | {write[k][0]:,.1f} | {traffic[k]:,} |")
        if case["unit"] == "bytes":
            md += ["", f"Per call ({' + '.join(case['call'])}): {rec['traffic_bytes_per_call']:,} bytes of HBM traffic "
                   f"against {alg:,} algorithmic bytes (ratio {rec['traffic_over_algorithmic']:.4f}); the call's "
                   f"kernels take {call_us:.2f} us together = {rec['call_kernels_gbs']:,.1f} GB/s of algorithmic bytes "
                   f"({100 * rec['call_kernels_gbs'] / HBM_PEAK_GBS:.1f} % of 8 TB/s)."]
        else:
            md += ["", f"Per call: {rec['traffic_bytes_per_call']:,} bytes of HBM traffic in {call_us:.2f} us = "
                   f"{rec['hbm_gbs']:,.1f} GB/s ({100 * rec['hbm_gbs'] / HBM_PEAK_GBS:.1f} % of 8 TB/s): the K/V "
                   "re-reads of the query tiles of one request are served by the L2 caches."]
        if "read_pages_kernel" in kav:
            pb = traffic["read_pages_kernel"]
            rec["read_probe_gbs"] = round(pb / (kav["read_pages_kernel"] * 1e-6) / 1e9, 1)
            md += ["", f"Read probe: {pb:,} bytes counted per dispatch in {kav['read_pages_kernel']:.2f} us = "
                   f"{rec['read_probe_gbs']:,.1f} GB/s, the streaming-read rate of this page-gather shape."]
    if case.get("sq"):
        rs = list(csv.DictReader(open(os.path.join(d + "_sq", "run_counter_collection.csv"))))
        key = case["call"][0]
        per = {}
        for r in rs:
            if key in r["Kernel_Name"]:
                per.setdefault(int(r["Dispatch_Id"]), {}).setdefault(r["Counter_Name"], 0.0)
                per[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
        names = SQ_COUNTERS.split()
        mean = {c: sum(v[c] for v in per.values()) / len(per) for c in names}
        simds, xcds = 1024, 8
        busy = (mean["SQ_VALU_MFMA_BUSY_CYCLES"] / simds) / (mean["GRBM_GUI_ACTIVE"] / xcds)
        rec.update({"sq_counters_mean_per_dispatch": {c: float(f"{mean[c]:.4g}") for c in names},
                    "mfma_busy": round(busy, 4),
                    "valu_per_mfma": round(mean["SQ_INSTS_VALU"] / mean["SQ_INSTS_MFMA"], 2),
                    "lds_per_mfma": round(mean["SQ_INSTS_LDS"] / mean["SQ_INSTS_MFMA"], 2),
                    "wait_inst_any_frac": round(mean["SQ_WAIT_INST_ANY"] / mean["SQ_WAVE_CYCLES"], 4)})
        tf = alg / (kav[key] * 1e-6) / 1e12
        rec["kernel_tflops"] = round(tf, 1)
        md += ["", f"SQ counters, mean per dispatch over {len(per)} dispatches of `{key}`:", "",
               "| Counter | Value |", "|---|---|"]
        md += [f"| {c} | {mean[c]:.4g} |" for c in names]
        md += ["", f"Matrix cores busy = (SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs) / (GRBM_GUI_ACTIVE / 8 XCDs) = "
               f"{100 * busy:.1f} %; vector instructions per matrix instruction {rec['valu_per_mfma']}; LDS "
               f"instructions per matrix instruction {rec['lds_per_mfma']}; SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES = "
               f"{100 * rec['wait_inst_any_frac']:.1f} %.", "",
               f"Work per call: {alg:.4g} flops of unmasked QK^T + PV; at the trace's average "
               f"{kav[key]:.1f} us the kernel runs at {tf:.1f} TFLOP/s ({100 * tf / BF16_PEAK_TFLOPS:.1f} % of "
               f"2.5 PFLOP/s dense bf16)."]
    md += ["", f"Kernel sources (SHA-256 in `{name}.json`; bench.py uses these figures only while they match): "
           + ", ".join(f"`{p}`" for p in case["sources"]) + "."]
    json.dump(rec, open(os.path.join(out_dir, name + ".json"), "w"), indent=1)
    open(os.path.join(out_dir, name + ".md"), "w").write("\n".join(md) + "\n")
    print(json.dumps(rec, indent=1))
    return rec


def bench_cascade(args):
    """Three BSR views (a prompt shared by all 64 requests, 16 group prefixes of 4, private
    suffixes) merged left to right, vs the single-level view over the same pages."""
    import torch
    from block_sparse_paged_bsr_amd import api
    import workloads as inputs

    b = inputs.cascade_decode(seed=0, poison=False)
    q, k, v = b.torch_values("cuda")
    C1 = api.query_num_workers("prefill", H_QO, H_KV, D)
    C2 = api.query_num_workers("decode", H_QO, H_KV, D)
    plans = []
    for qo, ip, ix, la in b.levels:
        mk = lambda C: api.Plan(ip, ix, la, num_pages=b.num_pages, num_qo_heads=H_QO, num_kv_heads=H_KV,
                                head_dim=D, page_size=b.page_size, qo_indptr=qo, causal=False, num_workers=C)
        # a level with little work (one prompt shared by every request) would be cut into
        # chunks of a few tokens at the full worker count: plan it for chunks of >= 256 tokens
        W = int(mk(C1).export()["total_work"])
        plans.append((mk(max(1, min(C1, (W + 255) // 256))), api.run_prefill))
    ip, ix, la = b.suffix
    plans.append((api.Plan(ip, ix, la, num_pages=b.num_pages, num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D,
                           page_size=b.page_size, num_workers=C2), api.run_decode))
    pf = api.Plan(*b.full, num_pages=b.num_pages, num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D,
                  page_size=b.page_size, num_workers=C2)
    wss = [api.alloc_workspace(p) for p, _ in plans]
    for (p, _), w in zip(plans, wss):
        p.upload(w)
    wf = api.alloc_workspace(pf)
    pf.upload(wf)
    R = q.shape[0]
    outs = [(torch.empty_like(q), torch.empty(R, H_QO, dtype=torch.float32, device="cuda")) for _ in plans]
    o = torch.empty_like(q)
    l = torch.empty(R, H_QO, dtype=torch.float32, device="cuda")
    pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(2)]

    def cascade(s):
        kk, vv = pools[s % 3]
        for ((p, fn), w, (oo, ll)) in zip(plans, wss, outs):
            fn(p, w, q, kk, vv, o=oo, lse=ll, sm_scale=SM)
        api.merge_state(outs[0][0], outs[0][1], outs[1][0], outs[1][1], o_out=o, lse_out=l)
        for oo, ll in outs[2:]:
            api.merge_state(o, l, oo, ll, o_out=o, lse_out=l)

    def single(s):
        kk, vv = pools[s % 3]
        api.run_decode(pf, wf, q, kk, vv, o=o, lse=l, sm_scale=SM)

    # all views in one composable plan: one attention launch and one merge launch
    cl = [dict(kv_indptr=ip_, kv_indices=ix_, last_page_len=la_, qo_indptr=qo_) for qo_, ip_, ix_, la_ in b.levels]
    cl.append(dict(kv_indptr=b.suffix[0], kv_indices=b.suffix[1], last_page_len=b.suffix[2]))
    cp = api.ComposablePlan(cl, num_pages=b.num_pages, num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D,
                            page_size=b.page_size, num_workers=C2)
    wcp = api.alloc_workspace(cp)
    cp.upload(wcp)

    def one_plan(s):
        kk, vv = pools[s % 3]
        api.run_prefill(cp, wcp, q, kk, vv, o=o, lse=l, sm_scale=SM)

    # the levels are independent until the fold: one stream each (default priority), joined
    # before the merges, so a small level does not leave the GPU idle while it runs
    streams = [torch.cuda.Stream() for _ in plans]

    def cascade_streams(s):
        kk, vv = pools[s % 3]
        cur = torch.cuda.current_stream()
        for st, (p, fn), w, (oo, ll) in zip(streams, plans, wss, outs):
            st.wait_stream(cur)
            with torch.cuda.stream(st):
                fn(p, w, q, kk, vv, o=oo, lse=ll, sm_scale=SM)
        for st in streams:
            cur.wait_stream(st)
        api.merge_state(outs[0][0], outs[0][1], outs[1][0], outs[1][1], o_out=o, lse_out=l)
        for oo, ll in outs[2:]:
            api.merge_state(o, l, oo, ll, o_out=o, lse_out=l)

    ms_p = time_calls(one_plan, args.steps, args.warmup)
    ms_pg = graph_replay_ms(one_plan, args.steps, args.warmup)
    ms_c = time_calls(cascade, args.steps, args.warmup)
    ms_cs = time_calls(cascade_streams, args.steps, args.warmup)
    ms_csg = graph_replay_ms(cascade_streams, args.steps, args.warmup)
    ms_s = time_calls(single, args.steps, args.warmup)
    # the cascade is several launches per step: replayed as one captured graph per KV pool
    # it is not bound by the host's per-call cost
    ms_cg = graph_replay_ms(cascade, args.steps, args.warmup)
    ms_sg = graph_replay_ms(single, args.steps, args.warmup)
    per = H_KV * D * 2 * 2
    qol = 2 * R * H_QO * D * 2 + R * H_QO * 4
    shared = sum(g_ * n_ for g_, n_ in zip(b.groups, b.prefix_lens))
    casc_bytes = shared * per + int(b.suffix_lens.sum()) * per + qol
    single_bytes = int((sum(b.prefix_lens) + b.suffix_lens).sum()) * per + qol
    return {"cascade_us": round(ms_p * 1e3, 2), "single_level_us": round(ms_s * 1e3, 2),
            "speedup": round(ms_s / ms_p, 3), "levels": len(plans), "one_plan_graph_us": round(ms_pg * 1e3, 2),
            "cascade_gbs_counted": round(casc_bytes / (ms_p * 1e-3) / 1e9, 1),
            "separate_plans_us": round(ms_c * 1e3, 2),
            "separate_plans_graph_us": round(ms_cg * 1e3, 2), "single_level_graph_us": round(ms_sg * 1e3, 2),
            "graph_speedup": round(ms_sg / ms_pg, 3),
            "cascade_streams_us": round(ms_cs * 1e3, 2), "cascade_streams_graph_us": round(ms_csg * 1e3, 2),
            "streams_graph_speedup": round(ms_sg / ms_csg, 3),
            "cascade_bytes": casc_bytes, "single_level_bytes": single_bytes,
            "single_level_gbs": round(single_bytes / (ms_s * 1e-3) / 1e9, 1)}


def bench_shared_prefix(args):
    """The shared-prefix kernel comparison of "FlashInfer: Making Attention Fit the Serving
    Workload" §7.3 (its Appendix Table 5): decode requests that share one prefix of P tokens
    and own 128-token suffixes, as two BSR views (the prefix as one block row of all queries,
    non-causal; the suffixes as ordinary decode) folded with merge_state, against the
    single-level view where every request reads prefix ++ suffix.  Shapes: batch 64 with
    P = 32,768 and batch 16 with P = 1,024.  The pages report 4090 -> 254.54 us and
    46.52 -> 45.17 us on their GPU: context, not the target.  The batch-64 shape rotates three
    copies of its KV pool (168 MB each, the composed path's whole read would otherwise stay in the
    last-level cache between calls); the batch-16 pool (13 MB) fits in that cache however many
    copies are rotated, so that shape runs on warm caches.  The composed and single-level outputs
    are compared with each other here; tests/test_gpu_shared_prefix.py checks both shapes against
    the oracle."""
    import torch
    from block_sparse_paged_bsr_amd import api
    import workloads as inputs

    out = {}
    for R, P in ((64, 32768), (16, 1024)):
        b = inputs.cascade_decode(seed=0, requests=R, groups=(1,), prefix_lens=(P,), suffix_lo=128,
                                  suffix_hi=128, poison=False)
        q, k, v = b.torch_values("cuda")
        pools = [(k, v)] + ([(k.clone(), v.clone()) for _ in range(2)] if R == 64 else [])
        qo, ip, ix, la = b.levels[0]
        C1 = api.query_num_workers("prefill", H_QO, H_KV, D)
        C2 = api.query_num_workers("decode", H_QO, H_KV, D)
        mk = lambda C: api.Plan(ip, ix, la, num_pages=b.num_pages, num_qo_heads=H_QO, num_kv_heads=H_KV,
                                head_dim=D, page_size=b.page_size, qo_indptr=qo, causal=False, num_workers=C)
        # chunks of >= 256 keys for the prefix level (see bench_cascade)
        W = int(mk(C1).export()["total_work"])
        p1 = mk(max(1, min(C1, (W + 255) // 256)))
        sip, six, sla = b.suffix
        p2 = api.Plan(sip, six, sla, num_pages=b.num_pages, num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D,
                      page_size=b.page_size, num_workers=C2)
        pf = api.Plan(*b.full, num_pages=b.num_pages, num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D,
                      page_size=b.page_size, num_workers=C2)
        w1, w2, wf = api.alloc_workspace(p1), api.alloc_workspace(p2), api.alloc_workspace(pf)
        p1.upload(w1)
        p2.upload(w2)
        pf.upload(wf)
        o1, o2, o, of = (torch.empty_like(q) for _ in range(4))
        l1, l2, l, lf = (torch.empty(R, H_QO, dtype=torch.float32, device="cuda") for _ in range(4))

        def composed(s):
            kk, vv = pools[s % len(pools)]
            api.run_prefill(p1, w1, q, kk, vv, o=o1, lse=l1, sm_scale=SM)
            api.run_decode(p2, w2, q, kk, vv, o=o2, lse=l2, sm_scale=SM)
            api.merge_state(o1, l1, o2, l2, o_out=o, lse_out=l)

        def single(s):
            kk, vv = pools[s % len(pools)]
            api.run_decode(pf, wf, q, kk, vv, o=of, lse=lf, sm_scale=SM)

        # the same two views as one composable plan (16-row tiles of 4 queries on the decode kernel:
        # every tile reads the whole prefix, so this suits short prefixes)
        cp = api.ComposablePlan([dict(kv_indptr=ip, kv_indices=ix, last_page_len=la, qo_indptr=qo),
                                 dict(kv_indptr=sip, kv_indices=six, last_page_len=sla)],
                                num_pages=b.num_pages, num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D,
                                page_size=b.page_size, num_workers=C2)
        wc = api.alloc_workspace(cp)
        cp.upload(wc)
        oc, lc = torch.empty_like(q), torch.empty(R, H_QO, dtype=torch.float32, device="cuda")

        def one_plan(s):
            kk, vv = pools[s % len(pools)]
            api.run_prefill(cp, wc, q, kk, vv, o=oc, lse=lc, sm_scale=SM)

        steps = max(10, args.steps // 2)
        ms_p = time_calls(one_plan, steps, args.warmup)
        ms_pg = graph_replay_ms(one_plan, steps, args.warmup)
        ms_c = time_calls(composed, steps, args.warmup)
        ms_s = time_calls(single, steps, args.warmup)
        ms_cg = graph_replay_ms(composed, steps, args.warmup)
        ms_sg = graph_replay_ms(single, steps, args.warmup)
        composed(0)
        single(0)
        one_plan(0)
        torch.cuda.synchronize()
        diff = float((o.float() - of.float()).abs().max())
        diff_p = float((oc.float() - of.float()).abs().max())
        per = H_KV * D * 2 * 2
        out[f"batch{R}_prefix{P}"] = {
            "composed_us": round(ms_c * 1e3, 2), "composed_graph_us": round(ms_cg * 1e3, 2),
            "single_level_us": round(ms_s * 1e3, 2), "single_level_graph_us": round(ms_sg * 1e3, 2),
            "speedup": round(ms_s / ms_c, 2),
            # (the small shape's eager calls are bound by the host's per-call cost: compare graphs)
            "graph_speedup": round(ms_sg / ms_cg, 2),
            "composed_bytes": (P + R * 128) * per, "single_level_bytes": R * (P + 128) * per,
            "max_abs_diff_O_composed_vs_single": round(diff, 5),
            "composable_plan_us": round(ms_p * 1e3, 2), "composable_plan_graph_us": round(ms_pg * 1e3, 2),
            "composable_plan_speedup": round(ms_s / ms_p, 2),
            "max_abs_diff_O_composable_plan_vs_single": round(diff_p, 5)}
        log(f"shared prefix batch {R}, prefix {P}: composed {ms_c * 1e3:.1f} us (graph {ms_cg * 1e3:.1f}), "
            f"single level {ms_s * 1e3:.1f} us, max|O composed - O single| {diff:.2e}")
        del q, k, v, pools, o1, o2, o, of, oc, w1, w2, wf, wc
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="decode only, no CPU baseline")
    ap.add_argument("--only", choices=["decode", "prefill", "vector", "composable", "cascade", "shared_prefix",
                                       "variants", "e4m3"],
                    default=None)
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--profile-case", choices=sorted(PROFILE_CASES), default=None,
                    help="run one case's calls only (for the rocprofv3 runs of profile_commands)")
    ap.add_argument("--profile-out", default=None, help="with --profile-case: write the event-timed call average here")
    ap.add_argument("--profile-commands", choices=sorted(PROFILE_CASES), default=None,
                    help="print the rocprofv3 commands behind profiles/<name>.json")
    ap.add_argument("--summarize", choices=sorted(PROFILE_CASES), default=None,
                    help="write profiles/<name>.json and .md from rocprof_out/<name>_* (no GPU)")
    ap.add_argument("--isa-rates", default=None, metavar="OUT.md",
                    help="run the execution-rate probes of libbsr_probe.so, print them and write OUT.md")
    args = ap.parse_args()
    if args.profile_commands:
        print("\n".join(profile_commands(args.profile_commands)))
        return
    if args.summarize:
        summarize_profile(args.summarize)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: every GPU would run the same kernels on its own "
              "requests and KV heads, there is no cross-GPU step to time; use --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "cu_count": props.multi_processor_count,
              "hbm_gib": round(props.total_memory / 2**30, 1), "torch": torch.__version__,
              "hip": getattr(torch.version, "hip", None)}
    log(f"device: {device}")
    if args.isa_rates:
        print(json.dumps(isa_rates(args.isa_rates)), flush=True)
        return
    if args.copy_calib:
        copy_calibration()
    if args.profile_case:
        run_profile_case(args.profile_case, args)
        return
    if args.only == "prefill":
        pf = bench_prefill(args)
        log(f"prefill: {pf['ms']*1e3:.1f} us, {pf['tflops']:.1f} TFLOP/s")
        return
    if args.only == "vector":
        log(json.dumps(bench_vector_sparse(args)))
        return
    if args.only == "composable":
        log(json.dumps(bench_composable(args)))
        return
    if args.only == "cascade":
        log(json.dumps(bench_cascade(args)))
        return
    if args.only == "shared_prefix":
        log(json.dumps(bench_shared_prefix(args)))
        return
    if args.only == "variants":
        log(json.dumps(bench_variants(args)))
        return
    if args.only == "e4m3":
        log(json.dumps(bench_e4m3(args)))
        return
    dec = bench_decode(args)
    log(f"decode: {dec['ms']*1e3:.1f} us/step, {dec['gbs']:.0f} GB/s; graph replay {dec['graph_ms']*1e3:.1f} us/step")
    out = {
        "metric": METRIC,
        "value": round(dec["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) Q/K/V, random page permutation)",
        "config": {
            "workload": "batched paged decode bf16: batch 64, KV lengths U[512,8192], page size 16, "
                        "32 query / 8 KV heads, head_dim 128, split-KV with the split requests folded in the kernel",
            "tokens": dec["tokens"], "algorithmic_bytes": dec["bytes"],
            "num_workers": dec["num_workers"], "work_items": dec["items"],
            "partial_slots": dec["slots"], "plan_host_us": round(dec["plan_us"], 1),
            "plan_upload_us": round(dec["upload_us"], 2),
            "median_us": round(dec["median_ms"] * 1e3, 2), "min_us": round(dec["min_ms"] * 1e3, 2),
            "p90_us": round(dec["p90_ms"] * 1e3, 2),
            "pct_hbm_peak": round(100 * dec["gbs"] / HBM_PEAK_GBS, 2),
            "kv_pool_rotation": 3,
            "graph_replay_us": round(dec["graph_ms"] * 1e3, 2),
            "graph_replay_gbs": round(dec["bytes"] / (dec["graph_ms"] * 1e-3) / 1e9, 1),
            "device": device,
        },
    }
    # Roofline of the decode call: one call = one launch of the attention kernel, which also folds
    # the split requests' partial states, timed over the timed region with events on the stream it
    # runs on (no per-launch events).  The kernel's rocprofv3 average and the HBM counters come
    # from the committed summary (profiles/decode_batch64.json), reported only while the kernel
    # sources are unchanged; the read ceiling is measured in this run.
    rec = profile_record("decode_batch64")
    ceil = dec["read_ceiling"]
    out["roofline"] = {"bound": "hbm", "achieved": round(dec["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(dec["gbs"] / HBM_PEAK_GBS, 4),
                       "traffic": rec["traffic_bytes_per_call"] if rec else None,
                       # one launch: split requests are folded inside the attention kernel
                       "kernel": "attn_decode_bf16_kernel<128, false, false, true>",
                       "call_avg_us": round(dec["ms"] * 1e3, 2), "algorithmic_bytes": dec["bytes"],
                       # the same pages read in the same order by a kernel that does nothing else
                       "read_ceiling_gbs": ceil["gbs"], "read_ceiling": ceil,
                       "frac_of_read_ceiling": round(dec["gbs"] / ceil["gbs"], 4)}
    if rec:
        kav = rec["kernel_avg_us"]
        out["roofline"].update({
            "rocprof_kernel_avg_us": kav["attn_decode_bf16_kernel"],
            "rocprof_attention_kernel_frac": round(dec["bytes"] / (kav["attn_decode_bf16_kernel"] * 1e-6) / 1e9
                                                   / HBM_PEAK_GBS, 4),
            "traffic_over_algorithmic": rec["traffic_over_algorithmic"],
            "rocprof_read_probe_gbs": rec.get("read_probe_gbs")})
    if not args.quick:
        del dec["step"], dec["out"]
        pf = bench_prefill(args)
        log(f"prefill: {pf['ms']*1e3:.1f} us, {pf['tflops']:.1f} TFLOP/s")
        prec = profile_record("prefill_ragged")
        out["prefill"] = {"workload": "ragged causal prefill bf16: batch 16, q_len = kv_len U[256,4096], "
                                      "page size 16, 32/8 heads, head_dim 128",
                          "tflops": round(pf["tflops"], 2), "ms": round(pf["ms"], 4),
                          "pct_bf16_peak": round(100 * pf["tflops"] / BF16_PEAK_TFLOPS, 2),
                          "flops": pf["flops"], "num_workers": pf["num_workers"], "partial_slots": pf["slots"],
                          # the call is one kernel (no request is split at this size): its event-timed
                          # average over the timed region is the kernel's launch duration
                          "roofline": {"bound": "mfma", "achieved": round(pf["tflops"], 2),
                                       "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": round(pf["tflops"] / BF16_PEAK_TFLOPS, 4),
                                       "kernel": "attn_prefill128_bf16_kernel<128, 2, false>",
                                       "rocprof_kernel_avg_us": prec["kernel_avg_us"] if prec else None,
                                       "rocprof_kernel_tflops": prec.get("kernel_tflops") if prec else None,
                                       "mfma_busy": prec.get("mfma_busy") if prec else None,
                                       "valu_per_mfma": prec.get("valu_per_mfma") if prec else None}}
        out["prefill"]["cpu_baseline"] = cpu_baseline_prefill(pf)
        torch.cuda.empty_cache()
        vs = bench_vector_sparse(args)
        log(f"vector sparse: {vs}")
        out["vector_sparse"] = vs
        torch.cuda.empty_cache()
        cp = bench_composable(args)
        log(f"composable: {cp}")
        out["composable"] = cp
        torch.cuda.empty_cache()
        cc = bench_cascade(args)
        log(f"cascade: {cc}")
        out["cascade"] = cc
        torch.cuda.empty_cache()
        out["shared_prefix"] = bench_shared_prefix(args)
        torch.cuda.empty_cache()
        va = bench_variants(args)
        log(f"variants: {va}")
        out["variants"] = va
        torch.cuda.empty_cache()
        e8 = bench_e4m3(args)
        log(f"e4m3 decode: {e8}")
        out["decode_e4m3"] = e8
        out["cpu_baseline"] = cpu_baseline(dec)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
