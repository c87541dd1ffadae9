"""Helpers for the GPU parity tests: run the HIP path and the oracle on one batch."""
import math
import sys

import numpy as np

from block_sparse_paged_bsr_amd import api
from oracle import attention as A

TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-5, 1e-5)}  # (O max-abs, LSE max-abs)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make_plan(b, num_workers=64, tile_q=0, causal=None, qo_indptr="auto", window_left=-1, soft_cap=0.0):
    qo = b.qo_indptr if qo_indptr == "auto" else qo_indptr
    return api.Plan(
        b.kv_indptr, b.kv_indices, b.last_page_len, num_pages=b.num_pages,
        num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
        page_size=b.page_size, qo_indptr=qo, causal=b.causal if causal is None else causal,
        num_workers=num_workers, tile_q=tile_q, window_left=window_left, logits_soft_cap=soft_cap,
    )


def run_gpu(b, p, decode=None, tensors=None):
    import torch

    q, k, v = tensors if tensors is not None else b.torch_values("cuda")
    ws = api.alloc_workspace(p)
    p.upload(ws)
    fn = api.run_decode if (b.qo_indptr is None if decode is None else decode) else api.run_prefill
    o, lse = fn(p, ws, q, k, v, sm_scale=1.0 / math.sqrt(b.head_dim))
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy(), ws


def oracle(b, requests=None, query_subset=None, causal=None, window_left=-1, soft_cap=0.0):
    return A.batch_attention(
        b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, b.page_size,
        b.num_qo_heads, b.num_kv_heads, 1.0 / math.sqrt(b.head_dim), qo_indptr=b.qo_indptr,
        causal=b.causal if causal is None else causal, requests=requests, query_subset=query_subset,
        window_left=window_left, soft_cap=soft_cap,
    )


def compare(o_gpu, l_gpu, o_ref, l_ref, dtype, what=""):
    """Element-by-element comparison on the rows the oracle evaluated (non-NaN)."""
    to, tl = TOL[dtype]
    rows = ~np.isnan(l_ref)
    assert rows.any(), "nothing compared"
    og, orf = o_gpu[rows], o_ref[rows]
    lg, lr = l_gpu[rows], l_ref[rows]
    assert np.all(np.isfinite(og)), f"{what}: non-finite O on the GPU"
    # empty states must match exactly (O = 0, LSE = -inf)
    empty = np.isneginf(lr)
    assert np.array_equal(np.isneginf(lg), empty), f"{what}: empty-state mismatch"
    fin = ~empty
    eo = float(np.max(np.abs(og - orf))) if og.size else 0.0
    el = float(np.max(np.abs(lg[fin] - lr[fin]))) if fin.any() else 0.0
    log(f"    {what}: max|dO| = {eo:.3e} (tol {to}), max|dLSE| = {el:.3e} (tol {tl}), rows={int(rows.sum())}")
    assert eo <= to, f"{what}: O error {eo} > {to}"
    assert el <= tl, f"{what}: LSE error {el} > {tl}"
    return eo, el
