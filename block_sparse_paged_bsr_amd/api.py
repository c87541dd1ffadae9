"""Python binding of libbsr_attn: argument marshalling only.

Every step of the attention path runs in the HIP library; this module converts
numpy/torch arguments into the pointers and sizes of include/bsr_attn.h.  PyTorch
supplies device memory and the current stream.
"""
from __future__ import annotations

import ctypes as C
import math
from typing import Optional

import numpy as np

from . import _lib
from ._lib import check, lib


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a), dtype=np.int32)
    return a, a.ctypes.data_as(_lib.i32p)


def _stream(stream=None):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _dtype_code(t):
    import torch

    if t.dtype == torch.float32:
        return _lib.DTYPE_F32
    if t.dtype == torch.bfloat16:
        return _lib.DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _plan_desc(kv_indptr, kv_indices, last_page_len, *, num_pages, num_qo_heads, num_kv_heads, head_dim, page_size,
               qo_indptr=None, causal=False, num_workers=0, tile_q=0, alpha=2, beta=1, window_left=-1,
               logits_soft_cap=0.0):
    """A bsr_plan_desc and the int32 arrays it points to (keep them alive while it is used).
    kv_indices None: a contiguous cache (request i's pages are kv_indptr[i] .. kv_indptr[i+1] - 1)."""
    kv_indptr, p_ip = _i32(kv_indptr)
    if kv_indices is None:
        p_ix = C.cast(None, _lib.i32p)
    else:
        kv_indices, p_ix = _i32(kv_indices)
    last_page_len, p_last = _i32(last_page_len)
    if qo_indptr is not None:
        qo_indptr, p_qo = _i32(qo_indptr)
    else:
        p_qo = C.cast(None, _lib.i32p)
    d = _lib.PlanDesc(
        batch=len(kv_indptr) - 1,
        qo_indptr=p_qo,
        kv_indptr=p_ip,
        kv_indices=p_ix,
        last_page_len=p_last,
        num_pages=int(num_pages),
        num_qo_heads=int(num_qo_heads),
        num_kv_heads=int(num_kv_heads),
        head_dim=int(head_dim),
        page_size=int(page_size),
        causal=int(bool(causal)),
        num_workers=int(num_workers),
        tile_q=int(tile_q),
        alpha=int(alpha),
        beta=int(beta),
        # the ABI counts the window in keys (0 = none); window_left keeps the pages'
        # notation, keys left of the diagonal (-1 = none)
        window_size=int(window_left) + 1,
        logits_soft_cap=float(logits_soft_cap),
    )
    return d, (kv_indptr, kv_indices, last_page_len, qo_indptr)


class Plan:
    """Host plan: the load-balanced split-KV partition of one batch (bsr_plan_create).
    kv_indices=None plans a contiguous cache (the identity page table)."""

    def __init__(
        self,
        kv_indptr,
        kv_indices,
        last_page_len,
        *,
        num_pages: int,
        num_qo_heads: int,
        num_kv_heads: int,
        head_dim: int,
        page_size: int,
        qo_indptr=None,
        causal: bool = False,
        num_workers: int = 0,
        tile_q: int = 0,
        alpha: int = 2,
        beta: int = 1,
        window_left: int = -1,
        logits_soft_cap: float = 0.0,
    ):
        d, keep = _plan_desc(kv_indptr, kv_indices, last_page_len, num_pages=num_pages, num_qo_heads=num_qo_heads,
                             num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
                             qo_indptr=qo_indptr, causal=causal, num_workers=num_workers, tile_q=tile_q,
                             alpha=alpha, beta=beta, window_left=window_left, logits_soft_cap=logits_soft_cap)
        h = C.c_void_p()
        check(lib().bsr_plan_create(C.byref(d), C.byref(h)))
        self._init(h, num_qo_heads, num_kv_heads, head_dim, num_pages, page_size, qo_indptr is None,
                   len(keep[0]) - 1, None if qo_indptr is None else int(keep[3][-1]))

    def _init(self, h, num_qo_heads, num_kv_heads, head_dim, num_pages, page_size, decode, batch, total_q):
        self._h = h
        self.num_qo_heads = int(num_qo_heads)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        self.num_pages = int(num_pages)
        self.page_size = int(page_size)
        self.decode = decode
        self.batch = batch
        self.total_q = batch if total_q is None else total_q
        self._ws = None
        self._mask_bits = None

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                lib().bsr_plan_destroy(h)
            except Exception:
                pass
            self._h = None

    @property
    def handle(self):
        return self._h

    def workspace_bytes(self) -> int:
        n = C.c_size_t()
        check(lib().bsr_plan_workspace_bytes(self._h, C.byref(n)))
        return int(n.value)

    def upload(self, workspace, stream=None):
        """Copy the plan metadata into ``workspace`` (a device uint8 tensor)."""
        check(lib().bsr_plan_upload(self._h, C.c_void_p(workspace.data_ptr()),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))
        self._ws = workspace
        return workspace

    def export(self) -> dict:
        v = _lib.PlanView()
        check(lib().bsr_plan_export(self._h, C.byref(v)))

        def arr(ptr, n, cols=1, dt=np.int32):
            if n == 0:
                return np.zeros((0, cols) if cols > 1 else (0,), dtype=dt)
            a = np.ctypeslib.as_array(ptr, shape=(n * cols,)).copy().astype(dt)
            return a.reshape(n, cols) if cols > 1 else a

        C_ = v.num_workers
        nm = v.num_merge
        merge_ptr = arr(v.merge_ptr, nm + 1)
        return {
            "batch": v.batch,
            "group_size": v.group_size,
            "tile_q": v.tile_q,
            "num_workers": C_,
            "num_slots": v.num_slots,
            "total_work": v.total_work,
            "chunk_limit": v.chunk_limit,
            "tiles": arr(v.tiles, v.num_tiles, 5),
            "items": arr(v.items, v.num_items, 8),
            "queue_ptr": arr(v.queue_ptr, C_ + 1),
            "queue_items": arr(v.queue_items, v.num_items),
            "worker_cost": arr(v.worker_cost, C_, dt=np.int64),
            "merge_tiles": arr(v.merge_tiles, nm),
            "merge_ptr": merge_ptr,
            "merge_slots": arr(v.merge_slots, int(merge_ptr[-1]) if nm else 0),
            "tile_lo": arr(v.tile_lo, v.num_tiles),
            "window_left": v.window_left,
            "logits_soft_cap": v.logits_soft_cap,
            "custom_mask_bits": v.custom_mask_bits,
            "num_levels": v.num_levels,
            "level_req_start": arr(v.level_req_start, v.num_levels + 1) if v.level_req_start else None,
            "merge_row_off": (arr(v.merge_row_off, int(merge_ptr[-1]) if nm else 0)
                              if v.merge_row_off else None),
        }


class ComposablePlan(Plan):
    """bsr_plan_create_composable: several BSR views ("levels") of one KV pool over the same
    queries, scheduled as one plan whose run folds every query's states over the levels.

    ``levels``: one dict per level with kv_indptr, kv_indices, last_page_len and optionally
    qo_indptr (None: one query per request); the other arguments are shared by all levels."""

    def __init__(self, levels, *, num_pages, num_qo_heads, num_kv_heads, head_dim, page_size, num_workers=0,
                 alpha=2, beta=1, logits_soft_cap=0.0):
        descs, keep = [], []
        for lv in levels:
            d, k = _plan_desc(lv["kv_indptr"], lv["kv_indices"], lv["last_page_len"], num_pages=num_pages,
                              num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                              page_size=page_size, qo_indptr=lv.get("qo_indptr"), alpha=alpha, beta=beta,
                              logits_soft_cap=logits_soft_cap)
            descs.append(d)
            keep.append(k)
        arr_t = _lib.PlanDesc * len(descs)
        h = C.c_void_p()
        check(lib().bsr_plan_create_composable(arr_t(*descs), len(descs), int(num_workers), C.byref(h)))
        k0 = keep[0]
        total_q = (len(k0[0]) - 1) if k0[3] is None else int(k0[3][-1])
        self._init(h, num_qo_heads, num_kv_heads, head_dim, num_pages, page_size, False, total_q, total_q)
        self.num_levels = len(descs)


def plan(*args, **kw) -> Plan:
    return Plan(*args, **kw)


def alloc_workspace(p: Plan, device="cuda"):
    import torch

    return torch.empty(max(p.workspace_bytes(), 256), dtype=torch.uint8, device=device)


def _check_run_args(p: Plan, q, k_cache, v_cache, o, lse, kv_dtypes=None):
    """Reject, before any launch, arguments the kernels would read or write out of bounds:
    shapes against the plan (the cache must hold the plan's num_pages pages of page_size
    tokens), dtypes, then device placement and layout."""
    import torch

    want_q = (p.total_q, p.num_qo_heads, p.head_dim)
    if tuple(q.shape) != want_q or tuple(o.shape) != want_q:
        raise ValueError(f"q/o shapes {tuple(q.shape)}, {tuple(o.shape)} != {want_q}")
    if tuple(lse.shape) != (p.total_q, p.num_qo_heads):
        raise ValueError(f"lse shape {tuple(lse.shape)} != {(p.total_q, p.num_qo_heads)}")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dim() != 4 or tuple(t.shape[1:]) != (p.page_size, p.num_kv_heads, p.head_dim):
            raise ValueError(f"{name} shape {tuple(t.shape)} is not [num_pages, {p.page_size}, "
                             f"{p.num_kv_heads}, {p.head_dim}]")
        if t.shape[0] < p.num_pages:
            raise ValueError(f"{name} holds {t.shape[0]} pages, the plan indexes {p.num_pages}")
    if kv_dtypes is None:
        if not (q.dtype == k_cache.dtype == v_cache.dtype == o.dtype):
            raise TypeError("q/k/v/o must share one dtype")
    else:
        if q.dtype != torch.bfloat16 or o.dtype != torch.bfloat16:
            raise TypeError("q and o must be bfloat16")
        if k_cache.dtype not in kv_dtypes or v_cache.dtype != k_cache.dtype:
            raise TypeError("k_cache/v_cache must hold E4M3 bytes (uint8 or float8_e4m3fn)")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("o", o), ("lse", lse)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")


def _run(fn, p: Plan, ws, q, k_cache, v_cache, o, lse, sm_scale, stream):
    import torch

    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(p.head_dim)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[0], p.num_qo_heads, dtype=torch.float32, device=q.device)
    _check_run_args(p, q, k_cache, v_cache, o, lse)
    check(
        fn(
            p.handle,
            C.c_void_p(ws.data_ptr()),
            C.c_void_p(q.data_ptr()),
            C.c_void_p(k_cache.data_ptr()),
            C.c_void_p(v_cache.data_ptr()),
            C.c_void_p(o.data_ptr()),
            C.cast(C.c_void_p(lse.data_ptr()), C.POINTER(C.c_float)),
            _dtype_code(q),
            float(sm_scale),
            _stream(stream),
        )
    )
    return o, lse


def run_decode(p: Plan, ws, q, k_cache, v_cache, o=None, lse=None, sm_scale=None, stream=None):
    """bsr_run_decode: one query per request; returns (O, LSE)."""
    return _run(lib().bsr_run_decode, p, ws, q, k_cache, v_cache, o, lse, sm_scale, stream)


def run_decode_scratch(p: Plan, q, k_cache, v_cache, o, lse, sm_scale=None, stream=None):
    """bsr_run_decode_scratch: bsr_run_decode on the library's static scratch (no workspace, no
    allocation in the call; o and lse are the caller's)."""
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(p.head_dim)
    _check_run_args(p, q, k_cache, v_cache, o, lse)
    check(lib().bsr_run_decode_scratch(
        p.handle, C.c_void_p(q.data_ptr()), C.c_void_p(k_cache.data_ptr()), C.c_void_p(v_cache.data_ptr()),
        C.c_void_p(o.data_ptr()), C.cast(C.c_void_p(lse.data_ptr()), C.POINTER(C.c_float)), _dtype_code(q),
        float(sm_scale), _stream(stream)))
    return o, lse


def run_prefill(p: Plan, ws, q, k_cache, v_cache, o=None, lse=None, sm_scale=None, stream=None):
    """bsr_run_prefill: ragged (causal per plan) queries; returns (O, LSE)."""
    return _run(lib().bsr_run_prefill, p, ws, q, k_cache, v_cache, o, lse, sm_scale, stream)


def pack_custom_mask(masks) -> np.ndarray:
    """Pack per-request boolean matrices [l_qo, l_kv] (request order, row-major) into the
    bit string bsr_run_prefill_masked reads: bit b at bit b % 8 of byte b // 8."""
    flat = [np.asarray(m, dtype=bool).reshape(-1) for m in masks]
    allbits = np.concatenate(flat) if flat else np.zeros(0, dtype=bool)
    return np.packbits(allbits, bitorder="little")


def run_prefill_masked(p: Plan, ws, q, k_cache, v_cache, mask, o=None, lse=None, sm_scale=None, stream=None):
    """bsr_run_prefill_masked: ``mask`` is a uint8 device tensor from ``pack_custom_mask``."""
    import torch

    if mask.dtype != torch.uint8 or not mask.is_cuda or not mask.is_contiguous():
        raise TypeError("mask must be a contiguous uint8 device tensor")
    if p._mask_bits is None:
        p._mask_bits = int(p.export()["custom_mask_bits"])
    need = (p._mask_bits + 7) // 8
    if mask.numel() < need:
        raise ValueError(f"mask holds {mask.numel()} bytes, the plan needs {need}")
    mptr = C.c_void_p(mask.data_ptr())

    def fn(h, ws_, q_, k_, v_, o_, lse_, dt, sm, st):
        return lib().bsr_run_prefill_masked(h, ws_, q_, k_, v_, mptr, o_, lse_, dt, sm, st)

    return _run(fn, p, ws, q, k_cache, v_cache, o, lse, sm_scale, stream)


def run_decode_e4m3(p: Plan, ws, q, k_cache, v_cache, k_scale: float, v_scale: float, o=None, lse=None,
                    sm_scale=None, stream=None):
    """bsr_run_decode_e4m3: decode over E4M3 K/V bytes (uint8 tensors [num_pages, P, H_kv, d])
    with per-tensor scales; Q and O bf16; returns (O, LSE)."""
    import torch

    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(p.head_dim)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[0], p.num_qo_heads, dtype=torch.float32, device=q.device)
    _check_run_args(p, q, k_cache, v_cache, o, lse, kv_dtypes=(torch.uint8, torch.float8_e4m3fn))
    check(
        lib().bsr_run_decode_e4m3(
            p.handle, C.c_void_p(ws.data_ptr()), C.c_void_p(q.data_ptr()), C.c_void_p(k_cache.data_ptr()),
            C.c_void_p(v_cache.data_ptr()), C.c_void_p(o.data_ptr()),
            C.cast(C.c_void_p(lse.data_ptr()), C.POINTER(C.c_float)), float(sm_scale), float(k_scale),
            float(v_scale), _stream(stream),
        )
    )
    return o, lse


def merge_state(o_a, lse_a, o_b, lse_b, o_out=None, lse_out=None, stream=None):
    """bsr_merge_state: (O_a, LSE_a) (+) (O_b, LSE_b) for [rows, heads, d] states."""
    import torch

    if o_out is None:
        o_out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    if o_a.dim() != 3:
        raise ValueError("o_a must be [rows, heads, head_dim]")
    rows, heads, d = o_a.shape
    if o_b.shape != o_a.shape or o_out.shape != o_a.shape:
        raise ValueError("merge_state: o_a, o_b and o_out must have one shape")
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b), ("lse_out", lse_out)):
        if tuple(t.shape) != (rows, heads):
            raise ValueError(f"merge_state: {name} shape {tuple(t.shape)} != {(rows, heads)}")
        if t.dtype != torch.float32:
            raise TypeError(f"merge_state: {name} must be float32")
    if not (o_a.dtype == o_b.dtype == o_out.dtype):
        raise TypeError("merge_state: o_a, o_b and o_out must share one dtype")
    for t in (o_a, lse_a, o_b, lse_b, o_out, lse_out):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("merge_state arguments must be contiguous device tensors")
    fp = C.POINTER(C.c_float)
    check(
        lib().bsr_merge_state(
            C.c_void_p(o_a.data_ptr()), C.cast(C.c_void_p(lse_a.data_ptr()), fp),
            C.c_void_p(o_b.data_ptr()), C.cast(C.c_void_p(lse_b.data_ptr()), fp),
            C.c_void_p(o_out.data_ptr()), C.cast(C.c_void_p(lse_out.data_ptr()), fp),
            rows, heads, d, _dtype_code(o_a), _stream(stream),
        )
    )
    return o_out, lse_out


def debug_gather_rows(p: Plan, ws, total_tokens: int, stream=None):
    """bsr_debug_gather_rows: int64 physical row of every logical token."""
    import torch

    rows = torch.full((max(total_tokens, 1),), -1, dtype=torch.int64, device=ws.device)
    check(lib().bsr_debug_gather_rows(p.handle, C.c_void_p(ws.data_ptr()), C.c_void_p(rows.data_ptr()), _stream(stream)))
    return rows[:total_tokens]


def query_num_workers(kind: str, num_qo_heads: int, num_kv_heads: int, head_dim: int, device: int = 0) -> int:
    out = C.c_int32()
    k = {"decode": 0, "prefill": 1}[kind]
    check(lib().bsr_query_num_workers(device, k, num_qo_heads, num_kv_heads, head_dim, C.byref(out)))
    return int(out.value)


def timing_enable(on: bool = True):
    check(lib().bsr_timing_enable(1 if on else 0))


def timing_read():
    am, an, mm, mn = C.c_double(), C.c_int64(), C.c_double(), C.c_int64()
    check(lib().bsr_timing_read(C.byref(am), C.byref(an), C.byref(mm), C.byref(mn)))
    return {"attn_ms": am.value, "attn_launches": an.value, "merge_ms": mm.value, "merge_launches": mn.value}


def version() -> str:
    return lib().bsr_version().decode()
