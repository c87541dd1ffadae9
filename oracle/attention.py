"""Exact attention over a block-sparse (paged) KV cache, in float64, on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definitions followed, by page:

* Attention with a validity mask, S = Q K^T / sqrt(d) + M, O = softmax(S) V, with M
  zero where allowed and -inf where forbidden: "FlashInfer: Making Attention Fit the
  Serving Workload" (§2.1, eq. 1).  The score scale is a parameter ``sm_scale``
  (1/sqrt(d) for the standard operator).
* Attention state (O, LSE) of an index set, LSE = log of the sum of exp(scores):
  "FlashInfer 原理" (§④); "FlashInfer: Engineering a Customizable, Block-Sparse
  Attention Engine for LLM Inference Serving" (§III.2); review §3.1 (eqs. 4-5).
* Merge of two states with a shared maximum and an explicit empty-state rule:
  review §3.2 (eq. 6) and §3.3 (Algorithm 1).
* Page-table addressing, p = indices[floor(t / B_c)], t_phys = p B_c + t mod B_c:
  review §4.1 (eq. 7); the last page may be partly filled (review §4.1; last-page
  length in "FlashInfer: A Customizable Attention Engine for LLM Serving", §8).
* GQA: query head h reads KV head floor(h / g), g = H_qo / H_kv (review §2.2, eq. 3).
* Causal masks use logical positions, aligned bottom-right: query position q of a
  request with l_qo queries and l_kv keys may see key k iff k <= q + l_kv - l_qo
  (review §4.1; the sliding-window predicate in "FlashInfer 原理" §⑧ carries the same
  kv_len - qo_len offset).
* Variants ("FlashInfer 原理" §⑧; review §5, eq. 8): a sliding window of
  ``window_left`` keys lets query q see key k only if k >= q + l_kv - l_qo -
  window_left (the lower half of the §⑧ predicate; the causal flag supplies the upper
  half); a logits soft cap c > 0 replaces every score s = sm_scale q.k by c tanh(s / c)
  before the mask decides which scores take part.
* Custom masks ("FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for
  LLM Inference Serving" §VII, LogitsMask; tree and importance masks, §III.1): an arbitrary
  boolean matrix per request, [l_qo, l_kv], stored row-major as bits (bit b of the
  concatenation is bit b mod 8 of byte b div 8, requests one after another).  The pages
  do not fix a storage format; this packing is the plainest one.  A key takes part only
  if the custom mask and every other predicate (causal, window) allow it.

Nothing here tiles, fuses or reorders: the score matrix of every (request, head) is
materialised and each row goes through softmax on its own.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


# ---------------------------------------------------------------------------
# Paging: lengths and physical rows
# ---------------------------------------------------------------------------


def kv_lengths(kv_indptr, last_page_len, page_size):
    """l_kv of every request: (n - 1) * P + last when the request owns n > 0 pages.

    Review §4.1: the last physical page may hold unused slots, so the length comes
    from the page count and the last page's fill.
    """
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    last = np.asarray(last_page_len, dtype=np.int64)
    n = kv_indptr[1:] - kv_indptr[:-1]
    return np.where(n > 0, (n - 1) * page_size + last, 0)


def physical_rows(kv_indptr, kv_indices, last_page_len, page_size, i):
    """Physical token rows of request ``i`` in logical order (review §4.1, eq. 7)."""
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    l_kv = int(kv_lengths(kv_indptr[i : i + 2], np.asarray(last_page_len)[i : i + 1], page_size)[0])
    t = np.arange(l_kv, dtype=np.int64)
    pages = kv_indices[kv_indptr[i] + t // page_size]
    return pages * page_size + t % page_size


# ---------------------------------------------------------------------------
# Dense attention for one head: the plain definition (review eq. 1)
# ---------------------------------------------------------------------------


def attention_one_head(q, k, v, sm_scale, allowed=None, soft_cap=0.0):
    """O and LSE of one head: materialise S, softmax each row.

    q: [Lq, d], k: [Lk, d], v: [Lk, dv]; allowed: bool [Lq, Lk] or None (all allowed).
    soft_cap > 0 transforms the scores to soft_cap * tanh(S / soft_cap) (eq. 8) before
    masking.  A row with no allowed key is the empty state: O = 0, LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Lq, Lk = q.shape[0], k.shape[0]
    S = float(sm_scale) * (q @ k.T) if Lk > 0 else np.zeros((Lq, 0))
    if soft_cap > 0:
        S = float(soft_cap) * np.tanh(S / float(soft_cap))
    if allowed is not None:
        S = np.where(allowed, S, NEG_INF)
    O = np.zeros((Lq, v.shape[1]), dtype=np.float64)
    lse = np.full(Lq, NEG_INF, dtype=np.float64)
    for r in range(Lq):
        row = S[r]
        if row.size == 0:
            continue
        m = row.max()
        if m == NEG_INF:
            continue
        p = np.exp(row - m)
        Z = p.sum()
        O[r] = (p @ v) / Z
        lse[r] = m + math.log(Z)
    return O, lse


def causal_allowed(l_qo, l_kv):
    """Bottom-right aligned causal predicate on logical positions, [l_qo, l_kv]."""
    qpos = np.arange(l_qo)[:, None]
    kpos = np.arange(l_kv)[None, :]
    return kpos <= qpos + (l_kv - l_qo)


def window_allowed(l_qo, l_kv, window_left):
    """Sliding-window predicate ("FlashInfer 原理" §⑧): key k visible to query q iff
    k + l_qo + window_left >= l_kv + q, i.e. k >= q + l_kv - l_qo - window_left."""
    qpos = np.arange(l_qo)[:, None]
    kpos = np.arange(l_kv)[None, :]
    return kpos + l_qo + window_left >= l_kv + qpos


def unpack_custom_mask(bits, qo_lens, kv_lens):
    """Per-request bool matrices [l_qo, l_kv] from the packed bit string (module
    docstring): request i starts at bit sum_{r<i} l_qo(r) l_kv(r); inside a request,
    bit q * l_kv + k says whether query q may see key k."""
    bits = np.asarray(bits, dtype=np.uint8)
    out = []
    start = 0
    for lq, lk in zip(qo_lens, kv_lens):
        lq, lk = int(lq), int(lk)
        out_i = np.zeros((lq, lk), dtype=bool)
        for q in range(lq):
            for k in range(lk):
                b = start + q * lk + k
                out_i[q, k] = (int(bits[b // 8]) >> (b % 8)) & 1 == 1
        out.append(out_i)
        start += lq * lk
    return out


# ---------------------------------------------------------------------------
# Batched attention over a BSR / paged KV cache
# ---------------------------------------------------------------------------


def batch_attention(
    q,
    k_cache,
    v_cache,
    kv_indptr,
    kv_indices,
    last_page_len,
    page_size,
    num_qo_heads,
    num_kv_heads,
    sm_scale,
    qo_indptr=None,
    causal=False,
    requests=None,
    query_subset=None,
    window_left=-1,
    soft_cap=0.0,
    custom_mask=None,
):
    """Attention of every (query, head) of a ragged batch over its own paged KV.

    q: [total_q, H_qo, d]; k_cache, v_cache: [num_pages, P, H_kv, d] (any float
    dtype, upcast exactly to float64).  ``qo_indptr`` None means one query per
    request (decode).  Returns O [total_q, H_qo, d] and LSE [total_q, H_qo] in
    float64; only rows of ``requests`` (default all) are filled, the rest stay NaN.
    ``query_subset`` maps a request to the query positions (0-based within the
    request) to evaluate; each query row is independent of the others, so a subset
    is the same definition on fewer rows.  ``window_left`` >= 0 adds the sliding-window
    mask and ``soft_cap`` > 0 the score soft cap (module docstring).  ``custom_mask``: a
    list of per-request bool matrices [l_qo, l_kv] (``unpack_custom_mask``), ANDed with
    the other predicates.
    """
    assert num_qo_heads % num_kv_heads == 0
    g = num_qo_heads // num_kv_heads
    B = len(kv_indptr) - 1
    if qo_indptr is None:
        qo_indptr = np.arange(B + 1, dtype=np.int64)
    qo_indptr = np.asarray(qo_indptr, dtype=np.int64)
    d = q.shape[-1]
    H_kv = num_kv_heads
    k_flat = np.asarray(k_cache).reshape(-1, H_kv, d)
    v_flat = np.asarray(v_cache).reshape(-1, H_kv, v_cache.shape[-1])
    total_q = int(qo_indptr[-1])
    O = np.full((total_q, num_qo_heads, v_flat.shape[-1]), np.nan, dtype=np.float64)
    lse = np.full((total_q, num_qo_heads), np.nan, dtype=np.float64)
    reqs = range(B) if requests is None else requests
    for i in reqs:
        rows = physical_rows(kv_indptr, kv_indices, last_page_len, page_size, i)
        q0, q1 = int(qo_indptr[i]), int(qo_indptr[i + 1])
        l_qo, l_kv = q1 - q0, len(rows)
        sel = np.arange(l_qo)
        if query_subset is not None and i in query_subset:
            sel = np.asarray(query_subset[i], dtype=np.int64)
        allowed = causal_allowed(l_qo, l_kv) if causal else None
        if window_left >= 0:
            win = window_allowed(l_qo, l_kv, window_left)
            allowed = win if allowed is None else (allowed & win)
        if custom_mask is not None:
            cm = np.asarray(custom_mask[i], dtype=bool)
            assert cm.shape == (l_qo, l_kv)
            allowed = cm if allowed is None else (allowed & cm)
        if allowed is not None:
            allowed = allowed[sel]
        K_i = k_flat[rows].astype(np.float64)  # [l_kv, H_kv, d]
        V_i = v_flat[rows].astype(np.float64)
        for h in range(num_qo_heads):
            hk = h // g
            o, s = attention_one_head(
                q[q0 + sel, h].astype(np.float64), K_i[:, hk], V_i[:, hk], sm_scale, allowed, soft_cap
            )
            O[q0 + sel, h] = o
            lse[q0 + sel, h] = s
    return O, lse


# ---------------------------------------------------------------------------
# Attention state merge (review §3.2 eq. 6, §3.3 Algorithm 1)
# ---------------------------------------------------------------------------


def merge_state(o_a, lse_a, o_b, lse_b):
    """(O_A, l_A) (+) (O_B, l_B) for every row; last axis of O is the value dim.

    A state whose LSE is -inf is empty (no key).  Both empty -> empty; one empty ->
    the other passes through; otherwise the shared-maximum form of eq. 6.
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    o = np.zeros(np.broadcast(o_a, o_b).shape, dtype=np.float64)
    lse = np.full(np.broadcast(lse_a, lse_b).shape, NEG_INF, dtype=np.float64)
    for idx in np.ndindex(*lse.shape):
        la, lb = float(lse_a[idx]), float(lse_b[idx])
        va, vb = la != NEG_INF, lb != NEG_INF
        if not va and not vb:
            continue  # empty state: O = 0, LSE = -inf
        if va and not vb:
            o[idx], lse[idx] = o_a[idx], la
            continue
        if vb and not va:
            o[idx], lse[idx] = o_b[idx], lb
            continue
        m = max(la, lb)
        a = math.exp(la - m)
        b = math.exp(lb - m)
        o[idx] = (a * o_a[idx] + b * o_b[idx]) / (a + b)
        lse[idx] = m + math.log(a + b)
    return o, lse


def fold_states(states):
    """Left fold ((s0 (+) s1) (+) s2) ... over a list of (O, LSE) pairs."""
    o, l = states[0]
    for o2, l2 in states[1:]:
        o, l = merge_state(o, l, o2, l2)
    return o, l


def empty_state(shape_o):
    """The identity of the merge: O = 0, LSE = -inf."""
    return np.zeros(shape_o, dtype=np.float64), np.full(shape_o[:-1], NEG_INF)


# ---------------------------------------------------------------------------
# Composable two-level format (shared prefix + private suffix)
# ---------------------------------------------------------------------------


def composable_attention(
    q,
    k_cache,
    v_cache,
    level1,
    level2,
    page_size,
    num_qo_heads,
    num_kv_heads,
    sm_scale,
):
    """Attention over two BSR views of one KV pool, combined with the merge.

    ``level1`` = (qo_indptr, kv_indptr, kv_indices, last_page_len): each level-1
    "request" is a block row whose queries all read the same pages (a shared prefix,
    non-causal).  ``level2`` = (kv_indptr, kv_indices, last_page_len): one decode
    query per request over its private pages.  The decomposition and its merge follow
    "FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for LLM
    Inference Serving" (§IV.6) and "FlashInfer 原理" (§⑤).
    """
    qo1, ip1, ix1, la1 = level1
    ip2, ix2, la2 = level2
    o1, s1 = batch_attention(
        q, k_cache, v_cache, ip1, ix1, la1, page_size, num_qo_heads, num_kv_heads,
        sm_scale, qo_indptr=qo1, causal=False,
    )
    o2, s2 = batch_attention(
        q, k_cache, v_cache, ip2, ix2, la2, page_size, num_qo_heads, num_kv_heads,
        sm_scale, qo_indptr=None, causal=False,
    )
    o, s = merge_state(o1, s1, o2, s2)
    return o, s, (o1, s1), (o2, s2)


# ---------------------------------------------------------------------------
# Multi-level cascade: shared-prefix levels plus private suffixes
# ---------------------------------------------------------------------------


def cascade_attention(q, k_cache, v_cache, levels, suffix, page_size, num_qo_heads, num_kv_heads, sm_scale):
    """Attention over L + 1 BSR views of one KV pool folded left with the merge.

    ``levels``: per shared level, (qo_indptr, kv_indptr, kv_indices, last_page_len) whose
    block rows are groups of decode queries reading the same prefix pages (non-causal).
    ``suffix``: (kv_indptr, kv_indices, last_page_len), one query per request.  The
    multi-level cascade of "FlashInfer 原理" (§⑤: shared prefixes at several levels,
    recombined with merge_state); the fold order is level 0, 1, ..., suffix.
    Returns the folded (O, LSE) and the list of per-view states.
    """
    states = []
    for qo, ip, ix, la in levels:
        states.append(batch_attention(q, k_cache, v_cache, ip, ix, la, page_size, num_qo_heads,
                                      num_kv_heads, sm_scale, qo_indptr=qo, causal=False))
    ip, ix, la = suffix
    states.append(batch_attention(q, k_cache, v_cache, ip, ix, la, page_size, num_qo_heads,
                                  num_kv_heads, sm_scale, qo_indptr=None, causal=False))
    o, s = fold_states(states)
    return o, s, states
