"""Seeded synthetic workloads shared by the tests, the benchmark and the oracle checks
(a module of its own, outside the library package).

This module only *builds inputs*: request lengths, BSR page tables (``kv_indptr``,
``kv_indices``, ``last_page_len``), ragged query offsets and random Q/K/V values.
It holds none of the attention arithmetic, none of the planning logic and imports
neither the oracle nor the HIP library, so both sides can consume the same arrays.

Shapes follow the paged "NHD" layout of the plan/run workflow described in
"FlashInfer: A Customizable Attention Engine for LLM Serving" (§8): K and V are each
``[num_pages, page_size, num_kv_heads, head_dim]`` with the head dimension contiguous;
Q and O are ``[total_q, num_qo_heads, head_dim]``; queries are ragged (no padding)
and addressed through ``qo_indptr`` ("FlashInfer: Engineering a Customizable,
Block-Sparse Attention Engine for LLM Inference Serving", §IV.4).

Values are drawn as float32 N(0, 1) from ``numpy.random.default_rng(seed)`` and,
for bf16 workloads, rounded to bfloat16 with round-to-nearest-even (torch's
``.to(torch.bfloat16)``).  ``*_f32`` arrays hold exactly the rounded values, so the
oracle consumes the very numbers the GPU reads.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "PagedBatch",
    "page_table_from_lengths",
    "make_paged_batch",
    "tiny_decode_fp32",
    "batched_decode_bf16",
    "ragged_prefill_bf16",
    "vector_sparse_pair",
    "shared_prefix_decode",
    "E4m3Batch",
    "to_e4m3",
    "block_sparse_attention",
]


@dataclass
class PagedBatch:
    """One batch of paged attention inputs (host arrays + value tensors)."""

    page_size: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    qo_indptr: Optional[np.ndarray]  # int32[B+1] or None for decode (one query each)
    kv_indptr: np.ndarray  # int32[B+1]
    kv_indices: np.ndarray  # int32[nnz]
    last_page_len: np.ndarray  # int32[B]
    num_pages: int
    q_f32: np.ndarray  # float32 [total_q, H_qo, d] (exact copy of the device values)
    k_f32: np.ndarray  # float32 [num_pages, P, H_kv, d]
    v_f32: np.ndarray  # float32 [num_pages, P, H_kv, d]
    dtype: str  # "f32" or "bf16"
    kv_lens: np.ndarray = field(default=None)  # int32[B] generator-side lengths
    qo_lens: np.ndarray = field(default=None)  # int32[B]
    causal: bool = False
    name: str = ""

    @property
    def batch(self) -> int:
        return int(self.kv_indptr.shape[0] - 1)

    @property
    def total_q(self) -> int:
        return int(self.q_f32.shape[0])

    def torch_values(self, device="cpu"):
        """Q, K, V as torch tensors in the workload dtype (bf16 values are exact)."""
        import torch

        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        return tuple(
            torch.from_numpy(a).to(tdt).to(device) for a in (self.q_f32, self.k_f32, self.v_f32)
        )


def _round(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype and return them as float32."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).float().numpy()


def page_table_from_lengths(kv_lens, page_size, page_ids):
    """Build (kv_indptr, kv_indices, last_page_len) for requests of the given lengths.

    ``page_ids`` supplies the physical page of every logical page, in request order.
    A request of length 0 owns no page and gets last_page_len 0.
    """
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    npages = (kv_lens + page_size - 1) // page_size
    kv_indptr = np.zeros(len(kv_lens) + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(npages)
    last = np.where(npages > 0, kv_lens - (npages - 1) * page_size, 0).astype(np.int32)
    kv_indices = np.asarray(page_ids[: int(kv_indptr[-1])], dtype=np.int32)
    return kv_indptr, kv_indices, last


def make_paged_batch(
    seed: int,
    kv_lens,
    qo_lens=None,
    *,
    page_size: int,
    num_qo_heads: int,
    num_kv_heads: int,
    head_dim: int,
    dtype: str = "bf16",
    num_pages: Optional[int] = None,
    contiguous: bool = False,
    poison: bool = True,
    causal: bool = False,
    name: str = "",
    rng: Optional[np.random.Generator] = None,
) -> PagedBatch:
    """Random paged batch.  Physical pages are a random permutation of the pool.

    ``num_pages`` defaults to exactly the pages the batch needs.  With ``contiguous``
    the pages are handed out in order (request after request).  With ``poison`` the
    unused slots of last pages and every unreferenced page hold NaN, so any read
    outside the requests' tokens shows up in the outputs.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    B = len(kv_lens)
    need = int(((kv_lens + page_size - 1) // page_size).sum())
    pool = need if num_pages is None else int(num_pages)
    assert pool >= need
    if contiguous:
        page_ids = np.arange(need, dtype=np.int64)
    else:
        page_ids = rng.permutation(pool)[:need]
    kv_indptr, kv_indices, last = page_table_from_lengths(kv_lens, page_size, page_ids)

    if qo_lens is None:
        qo_indptr = None
        total_q = B
        qo_lens_arr = np.ones(B, dtype=np.int32)
    else:
        qo_lens_arr = np.asarray(qo_lens, dtype=np.int32)
        qo_indptr = np.zeros(B + 1, dtype=np.int32)
        qo_indptr[1:] = np.cumsum(qo_lens_arr)
        total_q = int(qo_indptr[-1])

    q = _round(rng.standard_normal((total_q, num_qo_heads, head_dim), dtype=np.float32), dtype)
    # Values of referenced tokens are drawn in logical order (request, token), so two
    # batches with the same seed and lengths but different page layouts hold the same
    # K/V contents token by token.
    ntok = int(kv_lens.sum())
    klog = _round(rng.standard_normal((ntok, num_kv_heads, head_dim), dtype=np.float32), dtype)
    vlog = _round(rng.standard_normal((ntok, num_kv_heads, head_dim), dtype=np.float32), dtype)
    fill = np.nan if poison else 0.0
    k = np.full((pool * page_size, num_kv_heads, head_dim), fill, dtype=np.float32)
    v = np.full((pool * page_size, num_kv_heads, head_dim), fill, dtype=np.float32)
    rows = _rows_for_fill(kv_indptr, kv_indices, last, page_size)
    k[rows] = klog
    v[rows] = vlog
    k = k.reshape(pool, page_size, num_kv_heads, head_dim)
    v = v.reshape(pool, page_size, num_kv_heads, head_dim)
    return PagedBatch(
        page_size=page_size,
        num_qo_heads=num_qo_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        qo_indptr=qo_indptr,
        kv_indptr=kv_indptr,
        kv_indices=kv_indices,
        last_page_len=last,
        num_pages=pool,
        q_f32=q,
        k_f32=k,
        v_f32=v,
        dtype=dtype,
        kv_lens=kv_lens.astype(np.int32),
        qo_lens=qo_lens_arr,
        causal=causal,
        name=name,
    )


def _rows_for_fill(kv_indptr, kv_indices, last, page_size):
    """Flat slot numbers of all referenced tokens in (request, token) order.

    This only places generated values into the pool; it is input construction, the
    oracle derives its own row addresses independently.
    """
    out = []
    for i in range(len(kv_indptr) - 1):
        pages = kv_indices[kv_indptr[i] : kv_indptr[i + 1]].astype(np.int64)
        if len(pages) == 0:
            continue
        slots = (pages[:, None] * page_size + np.arange(page_size)[None, :]).reshape(-1)
        n = (len(pages) - 1) * page_size + int(last[i])
        out.append(slots[:n])
    if not out:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(out)


# ---------------------------------------------------------------------------
# The five workloads.  Sizes follow the pages' serving shapes: decode with one
# query per request, page size 16 as in PagedAttention, head_dim 128, GQA 32/8,
# vector sparsity (page size 1) and a shared prefix with n = 4 parallel requests.
# ---------------------------------------------------------------------------


def tiny_decode_fp32(seed: int = 0, poison: bool = True) -> PagedBatch:
    """3 decode requests over 8 physical pages of 4 tokens, fp32, GQA 4/1, d=16.

    Page table of the three-request example in "FlashInfer 原理" (§⑤):
    indptr [0,3,4,6], indices [5,1,6,2,7,3]; last-page lengths [4,2,3].
    """
    rng = np.random.default_rng(seed)
    P, Hq, Hk, d = 4, 4, 1, 16
    kv_indptr = np.array([0, 3, 4, 6], dtype=np.int32)
    kv_indices = np.array([5, 1, 6, 2, 7, 3], dtype=np.int32)
    last = np.array([4, 2, 3], dtype=np.int32)
    kv_lens = np.array([12, 2, 7], dtype=np.int32)
    q = rng.standard_normal((3, Hq, d), dtype=np.float32)
    k = rng.standard_normal((8, P, Hk, d), dtype=np.float32)
    v = rng.standard_normal((8, P, Hk, d), dtype=np.float32)
    if poison:
        # Request 0 fills pages 5, 1, 6; request 1 uses slots 0-1 of page 2; request 2
        # fills page 7 and slots 0-2 of page 3.  Pages 0 and 4 are unreferenced.
        for arr in (k, v):
            arr[0] = np.nan
            arr[4] = np.nan
            arr[2, 2:] = np.nan
            arr[3, 3:] = np.nan
    return PagedBatch(
        page_size=P,
        num_qo_heads=Hq,
        num_kv_heads=Hk,
        head_dim=d,
        qo_indptr=None,
        kv_indptr=kv_indptr,
        kv_indices=kv_indices,
        last_page_len=last,
        num_pages=8,
        q_f32=q,
        k_f32=k,
        v_f32=v,
        dtype="f32",
        kv_lens=kv_lens,
        qo_lens=np.ones(3, dtype=np.int32),
        name="tiny_decode_fp32",
    )


def decode_lengths(seed: int, batch: int = 64, lo: int = 512, hi: int = 8192) -> np.ndarray:
    """KV lengths uniform in [lo, hi] (inclusive)."""
    return np.random.default_rng(seed).integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


def prefill_lengths(seed: int, batch: int = 16, lo: int = 256, hi: int = 4096) -> np.ndarray:
    """Query (= KV) lengths of the ragged prefill, uniform in [lo, hi] (inclusive)."""
    return np.random.default_rng(seed).integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


def batched_decode_bf16(
    seed: int = 0,
    batch: int = 64,
    kv_lo: int = 512,
    kv_hi: int = 8192,
    page_size: int = 16,
    num_qo_heads: int = 32,
    num_kv_heads: int = 8,
    head_dim: int = 128,
    poison: bool = True,
    dtype: str = "bf16",
) -> PagedBatch:
    """Batch-64 paged decode: KV lengths U[512, 8192], page size 16, 32/8 heads, d=128."""
    lens = decode_lengths(seed, batch, kv_lo, kv_hi)
    rng = np.random.default_rng(seed + 1000)
    return make_paged_batch(
        seed, lens, None, page_size=page_size, num_qo_heads=num_qo_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, dtype=dtype, poison=poison,
        name="batched_decode_bf16", rng=rng,
    )


def ragged_prefill_bf16(
    seed: int = 0,
    batch: int = 16,
    lo: int = 256,
    hi: int = 4096,
    page_size: int = 16,
    num_qo_heads: int = 32,
    num_kv_heads: int = 8,
    head_dim: int = 128,
    poison: bool = True,
    causal: bool = True,
    qo_lens=None,
) -> PagedBatch:
    """Ragged causal prefill: q_len = kv_len uniform in [256, 4096], page size 16."""
    lens = prefill_lengths(seed, batch, lo, hi)
    ql = lens if qo_lens is None else np.asarray(qo_lens, dtype=np.int32)
    rng = np.random.default_rng(seed + 2000)
    return make_paged_batch(
        seed, lens, ql, page_size=page_size, num_qo_heads=num_qo_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, dtype="bf16", poison=poison,
        causal=causal, name="ragged_prefill_bf16", rng=rng,
    )


def vector_sparse_pair(
    seed: int,
    kv_lens,
    qo_lens=None,
    *,
    pool_rows: int = 1 << 20,
    num_qo_heads: int = 32,
    num_kv_heads: int = 8,
    head_dim: int = 128,
    causal: bool = False,
    poison: bool = False,
):
    """Page size 1 batch scattered over a ``pool_rows`` pool, plus its contiguous twin.

    Both layouts hold identical K/V contents token by token and share Q: the twin's
    pool is the paged pool's referenced rows laid out request after request, with
    ``kv_indices`` = 0, 1, 2, ... (affine addressing).
    """
    import copy

    a = make_paged_batch(
        seed, kv_lens, qo_lens, page_size=1, num_qo_heads=num_qo_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, dtype="bf16", num_pages=pool_rows,
        poison=poison, causal=causal, name="vector_sparse_paged",
        rng=np.random.default_rng(seed + 3000),
    )
    b = copy.copy(a)
    ntok = int(np.asarray(kv_lens, dtype=np.int64).sum())
    rows_a = _rows_for_fill(a.kv_indptr, a.kv_indices, a.last_page_len, 1)
    b.kv_indices = np.arange(ntok, dtype=np.int32)
    b.k_f32 = a.k_f32.reshape(-1, num_kv_heads, head_dim)[rows_a].reshape(ntok, 1, num_kv_heads, head_dim)
    b.v_f32 = a.v_f32.reshape(-1, num_kv_heads, head_dim)[rows_a].reshape(ntok, 1, num_kv_heads, head_dim)
    b.num_pages = ntok
    b.name = "vector_sparse_contiguous"
    return a, b


@dataclass
class SharedPrefixBatch:
    """Two BSR views over one physical KV pool (shared prefix + per-request suffix)."""

    groups: int
    per_group: int
    prefix_len: int
    page_size: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    q_f32: np.ndarray  # [R, H_qo, d]
    k_f32: np.ndarray  # [num_pages, P, H_kv, d]
    v_f32: np.ndarray
    num_pages: int
    # level 1: one "request" per group, its per_group queries packed through qo_indptr
    l1_qo_indptr: np.ndarray
    l1_kv_indptr: np.ndarray
    l1_kv_indices: np.ndarray
    l1_last_page_len: np.ndarray
    # level 2: one request per query over its own suffix pages
    l2_kv_indptr: np.ndarray
    l2_kv_indices: np.ndarray
    l2_last_page_len: np.ndarray
    # single-level view (prefix ++ suffix per request), the uncomposed baseline
    full_kv_indptr: np.ndarray
    full_kv_indices: np.ndarray
    full_last_page_len: np.ndarray
    suffix_lens: np.ndarray
    dtype: str = "bf16"

    def torch_values(self, device="cpu"):
        import torch

        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        return tuple(
            torch.from_numpy(a).to(tdt).to(device) for a in (self.q_f32, self.k_f32, self.v_f32)
        )


def shared_prefix_decode(
    seed: int = 0,
    groups: int = 16,
    per_group: int = 4,
    prefix_len: int = 2048,
    suffix_lo: int = 128,
    suffix_hi: int = 1024,
    page_size: int = 16,
    num_qo_heads: int = 32,
    num_kv_heads: int = 8,
    head_dim: int = 128,
    poison: bool = True,
    dtype: str = "bf16",
) -> SharedPrefixBatch:
    """64 decode requests in 16 groups of 4 sharing a 2048-token prefix per group.

    The prefix of a group occupies full pages; every request owns distinct suffix
    pages; all pages come from one random permutation of the pool.  The decomposition
    into a shared block and private suffixes follows the composable-format discussion
    of "FlashInfer 原理" (§⑤) and of "FlashInfer: Engineering a Customizable,
    Block-Sparse Attention Engine for LLM Inference Serving" (§IV.6).
    """
    assert prefix_len % page_size == 0
    rng = np.random.default_rng(seed)
    R = groups * per_group
    suf = rng.integers(suffix_lo, suffix_hi, size=R, endpoint=True).astype(np.int32)
    pre_pages = prefix_len // page_size
    suf_pages = (suf + page_size - 1) // page_size
    pool = groups * pre_pages + int(suf_pages.sum())
    perm = rng.permutation(pool).astype(np.int64)
    pre_ids = perm[: groups * pre_pages].reshape(groups, pre_pages)
    suf_ids = perm[groups * pre_pages :]

    q = _round(rng.standard_normal((R, num_qo_heads, head_dim), dtype=np.float32), dtype)
    fill = np.nan if poison else 0.0
    k = np.full((pool, page_size, num_kv_heads, head_dim), fill, dtype=np.float32)
    v = np.full_like(k, fill)
    shape = (pre_pages, page_size, num_kv_heads, head_dim)
    for gi in range(groups):
        k[pre_ids[gi]] = _round(rng.standard_normal(shape, dtype=np.float32), dtype)
        v[pre_ids[gi]] = _round(rng.standard_normal(shape, dtype=np.float32), dtype)
    off = 0
    suf_lists = []
    for r in range(R):
        ids = suf_ids[off : off + suf_pages[r]]
        off += suf_pages[r]
        suf_lists.append(ids)
        n = int(suf[r])
        kk = _round(rng.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32), dtype)
        vv = _round(rng.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32), dtype)
        kf = k.reshape(-1, num_kv_heads, head_dim)
        vf = v.reshape(-1, num_kv_heads, head_dim)
        slots = (ids[:, None] * page_size + np.arange(page_size)[None, :]).reshape(-1)[:n]
        kf[slots] = kk
        vf[slots] = vv

    l1_qo = np.arange(0, R + 1, per_group, dtype=np.int32)
    l1_kv_indptr, l1_idx, l1_last = page_table_from_lengths(
        np.full(groups, prefix_len), page_size, pre_ids.reshape(-1)
    )
    l2_kv_indptr, l2_idx, l2_last = page_table_from_lengths(
        suf, page_size, np.concatenate(suf_lists) if suf_lists else np.zeros(0, np.int64)
    )
    full_ids = np.concatenate([np.concatenate([pre_ids[r // per_group], suf_lists[r]]) for r in range(R)])
    full_indptr, full_idx, full_last = page_table_from_lengths(
        prefix_len + suf.astype(np.int64), page_size, full_ids
    )
    return SharedPrefixBatch(
        groups=groups, per_group=per_group, prefix_len=prefix_len, page_size=page_size,
        num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        q_f32=q, k_f32=k, v_f32=v, num_pages=pool,
        l1_qo_indptr=l1_qo, l1_kv_indptr=l1_kv_indptr, l1_kv_indices=l1_idx,
        l1_last_page_len=l1_last, l2_kv_indptr=l2_kv_indptr, l2_kv_indices=l2_idx,
        l2_last_page_len=l2_last, full_kv_indptr=full_indptr, full_kv_indices=full_idx,
        full_last_page_len=full_last, suffix_lens=suf, dtype=dtype,
    )


@dataclass
class CascadeBatch:
    """L shared-prefix levels plus private suffixes: L + 1 BSR views over one KV pool.

    Level ``i`` < L groups the R decode requests into ``groups[i]`` block rows of
    R / groups[i] consecutive requests that share ``prefix_lens[i]`` tokens; a request's
    context is level 0's prefix, then level 1's, ..., then its own suffix.
    """

    groups: tuple
    prefix_lens: tuple
    page_size: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    q_f32: np.ndarray  # [R, H_qo, d]
    k_f32: np.ndarray  # [num_pages, P, H_kv, d]
    v_f32: np.ndarray
    num_pages: int
    levels: list  # per shared level: (qo_indptr, kv_indptr, kv_indices, last_page_len)
    suffix: tuple  # (kv_indptr, kv_indices, last_page_len), one request per query
    full: tuple  # single-level view: every request over all of its pages
    suffix_lens: np.ndarray
    dtype: str = "bf16"

    @property
    def requests(self):
        return int(self.q_f32.shape[0])

    def torch_values(self, device="cpu"):
        import torch

        tdt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        return tuple(
            torch.from_numpy(a).to(tdt).to(device) for a in (self.q_f32, self.k_f32, self.v_f32)
        )


def cascade_decode(
    seed: int = 0,
    requests: int = 64,
    groups=(1, 16),
    prefix_lens=(1024, 2048),
    suffix_lo: int = 128,
    suffix_hi: int = 1024,
    page_size: int = 16,
    num_qo_heads: int = 32,
    num_kv_heads: int = 8,
    head_dim: int = 128,
    poison: bool = True,
    dtype: str = "bf16",
) -> CascadeBatch:
    """Decode batch with a multi-level shared-prefix tree (the multi-level cascade of
    "FlashInfer 原理", §⑤ and §F2): by default one 1024-token prompt shared by all 64
    requests, 16 groups of 4 sharing a further 2048 tokens, and private suffixes
    U[128, 1024].  Prefixes occupy full pages; all pages come from one random
    permutation of the pool."""
    assert len(groups) == len(prefix_lens)
    rng = np.random.default_rng(seed)
    R = requests
    for g_, n_ in zip(groups, prefix_lens):
        assert R % g_ == 0 and n_ % page_size == 0
    suf = rng.integers(suffix_lo, suffix_hi, size=R, endpoint=True).astype(np.int32)
    lvl_pages = [g_ * (n_ // page_size) for g_, n_ in zip(groups, prefix_lens)]
    suf_pages = (suf + page_size - 1) // page_size
    pool = sum(lvl_pages) + int(suf_pages.sum())
    perm = rng.permutation(pool).astype(np.int64)
    q = _round(rng.standard_normal((R, num_qo_heads, head_dim), dtype=np.float32), dtype)
    fill = np.nan if poison else 0.0
    k = np.full((pool, page_size, num_kv_heads, head_dim), fill, dtype=np.float32)
    v = np.full_like(k, fill)
    kf = k.reshape(-1, num_kv_heads, head_dim)
    vf = v.reshape(-1, num_kv_heads, head_dim)

    def fill_tokens(ids, n):
        slots = (ids[:, None] * page_size + np.arange(page_size)[None, :]).reshape(-1)[:n]
        kf[slots] = _round(rng.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32), dtype)
        vf[slots] = _round(rng.standard_normal((n, num_kv_heads, head_dim), dtype=np.float32), dtype)

    off = 0
    levels, level_ids = [], []
    for g_, n_ in zip(groups, prefix_lens):
        npg = n_ // page_size
        ids = perm[off : off + g_ * npg].reshape(g_, npg)
        off += g_ * npg
        for gi in range(g_):
            fill_tokens(ids[gi], n_)
        qo = np.arange(0, R + 1, R // g_, dtype=np.int32)
        ip, ix, la = page_table_from_lengths(np.full(g_, n_), page_size, ids.reshape(-1))
        levels.append((qo, ip, ix, la))
        level_ids.append(ids)
    suf_lists = []
    for r in range(R):
        ids = perm[off : off + suf_pages[r]]
        off += suf_pages[r]
        suf_lists.append(ids)
        fill_tokens(ids, int(suf[r]))
    suffix = page_table_from_lengths(suf, page_size, np.concatenate(suf_lists))
    full_ids = np.concatenate([
        np.concatenate([level_ids[li][r // (R // g_)] for li, g_ in enumerate(groups)] + [suf_lists[r]])
        for r in range(R)])
    full = page_table_from_lengths(sum(prefix_lens) + suf.astype(np.int64), page_size, full_ids)
    return CascadeBatch(
        groups=tuple(groups), prefix_lens=tuple(prefix_lens), page_size=page_size,
        num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        q_f32=q, k_f32=k, v_f32=v, num_pages=pool, levels=levels, suffix=suffix, full=full,
        suffix_lens=suf, dtype=dtype,
    )


@dataclass
class E4m3Batch:
    """A paged batch whose K and V are stored as E4M3 bytes (OCP "FN" encoding) with one
    float scale per tensor: byte b stands for value(b) * scale.  Q stays in the base
    batch's dtype."""

    base: PagedBatch
    k_bytes: np.ndarray  # uint8 [num_pages, P, H_kv, d]
    v_bytes: np.ndarray  # uint8 [num_pages, P, H_kv, d]
    k_scale: float
    v_scale: float

    def torch_values(self, device="cpu"):
        """Q (base dtype), K and V bytes (uint8) as torch tensors."""
        import torch

        q = self.base.torch_values(device)[0]
        return q, torch.from_numpy(self.k_bytes).to(device), torch.from_numpy(self.v_bytes).to(device)


def to_e4m3(b: PagedBatch, k_scale: Optional[float] = None, v_scale: Optional[float] = None) -> E4m3Batch:
    """Store a batch's K and V as E4M3 bytes.

    Default scales are the per-tensor amax / 448 of the referenced tokens (so the largest
    value lands on the format's largest finite value); the bytes are torch's
    float8_e4m3fn rounding (nearest even) of value / scale, clamped to +-448.  Unused
    (poisoned) slots stay NaN (byte 0x7f).  Input construction only: the oracle decodes
    the bytes with its own decoder.
    """
    import torch

    def enc(x, scale):
        finite = np.isfinite(x)
        amax = float(np.max(np.abs(x[finite]))) if finite.any() else 1.0
        sc = float(scale) if scale is not None else (amax / 448.0 if amax > 0 else 1.0)
        y = np.clip(x / np.float32(sc), -448.0, 448.0)  # NaN stays NaN
        t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.float8_e4m3fn)
        return t.view(torch.uint8).numpy().copy(), sc

    kb, ks = enc(b.k_f32, k_scale)
    vb, vs = enc(b.v_f32, v_scale)
    return E4m3Batch(base=b, k_bytes=kb, v_bytes=vb, k_scale=ks, v_scale=vs)


@dataclass
class BlockSparseBatch:
    """Block-sparse attention over one dense sequence, as a BSR matrix of B_r x B_c blocks.

    ``dense`` holds Q [L, H_qo, d] and K/V as pages of B_c rows ([L / B_c, B_c, H_kv, d], page j
    = rows j B_c .. (j+1) B_c - 1); ``block_mask`` [L / B_r, L / B_c] says which blocks are
    present.  The BSR view: block row i is one "request" with the B_r queries of rows
    i B_r .. (i+1) B_r - 1 (``qo_indptr``) whose KV pages are the present column blocks in
    increasing order (``kv_indptr``, ``kv_indices``, full last pages).
    """

    dense: PagedBatch
    block_mask: np.ndarray
    block_r: int
    block_c: int


def block_sparse_attention(seed: int, L: int, block_r: int, block_c: int, density: float, *, num_qo_heads: int,
                           num_kv_heads: int, head_dim: int, dtype: str = "bf16") -> BlockSparseBatch:
    """Random block-sparse layout (each block present with probability ``density``; some
    block rows may be empty) over seeded N(0, 1) values."""
    assert L % block_r == 0 and L % block_c == 0
    rng = np.random.default_rng(seed)
    nr, nc = L // block_r, L // block_c
    bm = rng.random((nr, nc)) < density
    q = _round(rng.standard_normal((L, num_qo_heads, head_dim), dtype=np.float32), dtype)
    k = _round(rng.standard_normal((nc, block_c, num_kv_heads, head_dim), dtype=np.float32), dtype)
    v = _round(rng.standard_normal((nc, block_c, num_kv_heads, head_dim), dtype=np.float32), dtype)
    cols = [np.nonzero(bm[i])[0] for i in range(nr)]
    kv_indptr = np.zeros(nr + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum([len(c) for c in cols])
    kv_indices = np.concatenate(cols).astype(np.int32) if kv_indptr[-1] else np.zeros(0, dtype=np.int32)
    last = np.array([block_c if len(c) else 0 for c in cols], dtype=np.int32)
    qo_indptr = (np.arange(nr + 1) * block_r).astype(np.int32)
    pb = PagedBatch(page_size=block_c, num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                    qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices, last_page_len=last,
                    num_pages=nc, q_f32=q, k_f32=k, v_f32=v, dtype=dtype,
                    kv_lens=(kv_indptr[1:] - kv_indptr[:-1]) * block_c, qo_lens=np.full(nr, block_r, np.int32),
                    causal=False, name="block_sparse")
    return BlockSparseBatch(dense=pb, block_mask=bm, block_r=block_r, block_c=block_c)
