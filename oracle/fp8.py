"""Attention over an 8-bit float (E4M3) paged KV cache, in float64, on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages run decode with an e4m3 KV cache ("FlashInfer: Making Attention Fit the
Serving Workload", the vLLM integration of Appendix G.4, Table 8) but do not define the
encoding or its scaling.  Readings taken:

* E4M3 is the "FN" format of the OCP 8-bit floating point specification: one sign bit,
  four exponent bits with bias 7, three mantissa bits; exponent 0 holds the subnormals
  m/8 * 2^-6; the pattern S.1111.111 is NaN and there is no infinity, so the largest
  finite value is 1.75 * 2^8 = 448.
* Each of K and V carries one per-tensor float scale: a stored byte b stands for
  decode(b) * scale.  Scale 1 is plain e4m3.
* Everything else (queries, mask, softmax, output) is the attention of
  ``oracle.attention.batch_attention`` on the decoded, scaled values.

``e4m3_to_float`` writes the format definition out bit field by bit field (no table
taken from a library), so the tests can pin it against closed-form values and against
torch's own float8_e4m3fn conversion.
"""
from __future__ import annotations

import numpy as np

from oracle import attention as A


def e4m3_to_float(b) -> np.ndarray:
    """Value of every E4M3 (FN) byte in ``b`` as float64 (NaN for S.1111.111)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    v = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & (b & 0x7 == 7), np.nan, v)


def paged_decode_e4m3(q, k_bytes, v_bytes, k_scale, v_scale, kv_indptr, kv_indices, last_page_len,
                      page_size, num_qo_heads, num_kv_heads, sm_scale, requests=None):
    """Decode attention (one query per request) over e4m3 K and V bytes
    [num_pages, P, H_kv, d] with per-tensor scales; returns (O, LSE) in float64, rows of
    requests not in ``requests`` (default all) left NaN.  Each request's own pages are
    decoded on their own, so the whole pool is never expanded to float64."""
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    kv_indices = np.asarray(kv_indices, dtype=np.int64)
    B = len(kv_indptr) - 1
    d = q.shape[-1]
    O = np.full((B, num_qo_heads, v_bytes.shape[-1]), np.nan, dtype=np.float64)
    lse = np.full((B, num_qo_heads), np.nan, dtype=np.float64)
    for i in (range(B) if requests is None else requests):
        pages = kv_indices[kv_indptr[i]:kv_indptr[i + 1]]
        n = len(pages)
        k = e4m3_to_float(k_bytes[pages]) * float(k_scale)
        v = e4m3_to_float(v_bytes[pages]) * float(v_scale)
        o_i, l_i = A.batch_attention(q[i:i + 1], k.reshape(n, page_size, num_kv_heads, d),
                                     v.reshape(n, page_size, num_kv_heads, v_bytes.shape[-1]), [0, n], np.arange(n),
                                     [last_page_len[i]], page_size, num_qo_heads, num_kv_heads, sm_scale)
        O[i], lse[i] = o_i[0], l_i[0]
    return O, lse
