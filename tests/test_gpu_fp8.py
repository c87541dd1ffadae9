"""GPU parity of decode over an E4M3 KV cache (bsr_run_decode_e4m3) against the oracle of
``oracle/fp8.py``: the oracle decodes the very bytes the GPU reads, with its own decoder,
and applies the per-tensor scales in float64.  Tolerances are those of bf16 decode (the
kernel widens E4M3 to bf16 exactly, so the arithmetic is the bf16 path's)."""
import math

import numpy as np
import pytest

import workloads as I
from oracle import fp8
from tests.gpu_helpers import compare, log, make_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_paged_bsr_amd import api

    api.version()  # loads the library or raises


def _run(e, p, tensors=None):
    import torch
    from block_sparse_paged_bsr_amd import api

    b = e.base
    q, k, v = tensors if tensors is not None else e.torch_values("cuda")
    ws = api.alloc_workspace(p)
    p.upload(ws)
    o, lse = api.run_decode_e4m3(p, ws, q, k, v, e.k_scale, e.v_scale, sm_scale=1.0 / math.sqrt(b.head_dim))
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _oracle(e, requests=None, window_left=-1, soft_cap=0.0):
    b = e.base
    if window_left >= 0 or soft_cap > 0:
        from oracle import attention as A

        k = fp8.e4m3_to_float(e.k_bytes) * e.k_scale
        v = fp8.e4m3_to_float(e.v_bytes) * e.v_scale
        return A.batch_attention(b.q_f32, k, v, b.kv_indptr, b.kv_indices, b.last_page_len, b.page_size,
                                 b.num_qo_heads, b.num_kv_heads, 1.0 / math.sqrt(b.head_dim),
                                 requests=requests, window_left=window_left, soft_cap=soft_cap)
    return fp8.paged_decode_e4m3(b.q_f32, e.k_bytes, e.v_bytes, e.k_scale, e.v_scale, b.kv_indptr,
                                 b.kv_indices, b.last_page_len, b.page_size, b.num_qo_heads, b.num_kv_heads,
                                 1.0 / math.sqrt(b.head_dim), requests=requests)


CASES = [
    # (lens, P, Hq, Hk, d, workers, k_scale, v_scale)   (None: amax / 448)
    ([37, 1, 200, 16, 513], 16, 32, 8, 128, 8, None, None),
    ([37, 1, 200, 16, 513], 16, 32, 8, 128, 1, None, None),
    ([100, 0, 260, 31], 4, 8, 8, 128, 5, 0.02, 0.05),
    ([333, 70, 1], 1, 16, 4, 64, 6, None, None),
    ([129, 300], 16, 16, 2, 128, 7, 1.0, 1.0),   # g = 8, unit scales (values saturate at 448)
    ([1000, 17], 12, 16, 1, 64, 9, None, None),  # g = 16, page size 12
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_decode_e4m3_small(case):
    lens, P, Hq, Hk, d, C_, ks, vs = CASES[case]
    log(f"[decode_e4m3_small] lens={lens} P={P} H={Hq}/{Hk} d={d} workers={C_} scales={ks},{vs}")
    b = I.make_paged_batch(600 + case, lens, None, page_size=P, num_qo_heads=Hq, num_kv_heads=Hk,
                           head_dim=d, num_pages=sum((x + P - 1) // P for x in lens) + 7)
    e = I.to_e4m3(b, ks, vs)
    p = make_plan(b, num_workers=C_)
    o, l = _run(e, p)
    ro, rl = _oracle(e)
    compare(o, l, ro, rl, "bf16", "decode e4m3 small")


def test_decode_e4m3_with_window_and_cap():
    lens = [37, 1, 200, 16, 513]
    log(f"[decode_e4m3_variants] lens={lens} window=100 cap=3")
    b = I.make_paged_batch(650, lens, None, page_size=16, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                           num_pages=60)
    e = I.to_e4m3(b)
    p = make_plan(b, num_workers=6, window_left=100, soft_cap=3.0)
    o, l = _run(e, p)
    ro, rl = _oracle(e, window_left=100, soft_cap=3.0)
    compare(o, l, ro, rl, "bf16", "decode e4m3 window+cap")


def test_decode_e4m3_batch64_full():
    """Batch-64 paged decode at its full size over E4M3 K/V: every request against the oracle,
    two runs bitwise equal, and each call one launch (its 55 split requests folded inside the
    attention kernel, no merge launch)."""
    import torch
    from block_sparse_paged_bsr_amd import api

    b = I.batched_decode_bf16(seed=0)
    e = I.to_e4m3(b)
    C_ = api.query_num_workers("decode", 32, 8, 128)
    log(f"[decode_e4m3_batch64_full] tokens={int(b.kv_lens.sum())} workers={C_} scales={e.k_scale:.4g},{e.v_scale:.4g}")
    p = make_plan(b, num_workers=C_)
    tens = e.torch_values("cuda")
    api.timing_enable(True)
    try:
        o, l = _run(e, p, tens)
        o2, l2 = _run(e, p, tens)
        t = api.timing_read()
    finally:
        api.timing_enable(False)
    assert t["attn_launches"] == 2 and t["merge_launches"] == 0, t
    ro, rl = _oracle(e)
    compare(o, l, ro, rl, "bf16", "decode e4m3 batch64")
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    torch.cuda.synchronize()


def test_decode_e4m3_rejects_what_it_does_not_serve():
    import torch
    from block_sparse_paged_bsr_amd import _lib, api

    b = I.make_paged_batch(660, [40, 9], None, page_size=16, num_qo_heads=32, num_kv_heads=1, head_dim=128)
    e = I.to_e4m3(b)
    p = make_plan(b, num_workers=4)  # g = 32: more query heads per KV head than the kernel serves
    ws = api.alloc_workspace(p)
    p.upload(ws)
    q, k, v = e.torch_values("cuda")
    with pytest.raises(_lib.BsrError) as ei:
        api.run_decode_e4m3(p, ws, q, k, v, e.k_scale, e.v_scale)
    assert ei.value.status == _lib.BSR_UNSUPPORTED
    b2 = I.make_paged_batch(661, [40, 9], None, page_size=16, num_qo_heads=8, num_kv_heads=2, head_dim=128)
    e2 = I.to_e4m3(b2)
    p2 = make_plan(b2, num_workers=4)
    ws2 = api.alloc_workspace(p2)
    p2.upload(ws2)
    q2, k2, v2 = e2.torch_values("cuda")
    for ks, vs in ((0.0, 1.0), (1.0, float("nan")), (float("inf"), 1.0)):
        with pytest.raises(_lib.BsrError) as ei:
            api.run_decode_e4m3(p2, ws2, q2, k2, v2, ks, vs)
        assert ei.value.status == _lib.BSR_INVALID_ARG
    torch.cuda.synchronize()
