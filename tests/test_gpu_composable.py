"""GPU parity of composable plans (bsr_plan_create_composable): several BSR views of one KV pool
scheduled as one plan -- one attention launch over every view's block rows on the decode kernel
(query tiles of 16 packed rows), one merge launch folding each query's states over the views --
against the fp64 oracle's attention over the union of the views' keys and its per-view fold.
Also the decode kernel on non-causal tiles of several queries through ordinary plans.

Tolerances: bf16 inputs with fp32 accumulation -> O max-abs 2e-2, LSE max-abs 1e-2.
"""
import math

import numpy as np
import pytest

import workloads as I
from oracle import attention as A
from tests.gpu_helpers import compare, log, make_plan, oracle, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_paged_bsr_amd import api

    api.version()  # loads the library or raises


def _run_composable(levels, b, q, k, v, num_workers=256):
    import torch
    from block_sparse_paged_bsr_amd import api

    p = api.ComposablePlan(levels, num_pages=b.num_pages, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                           page_size=b.page_size, num_workers=num_workers)
    ws = api.alloc_workspace(p)
    p.upload(ws)
    o, l = api.run_prefill(p, ws, q, k, v, sm_scale=1.0 / math.sqrt(128))
    o2, l2 = api.run_prefill(p, ws, q, k, v, sm_scale=1.0 / math.sqrt(128))
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(l, l2)  # run twice: bitwise identical
    return p, o.float().cpu().numpy(), l.cpu().numpy()


def test_composable_shared_prefix_one_plan():
    """16 groups of 4 requests sharing a 2048-token prefix (one block row of 4 queries per group)
    plus private suffixes U[128, 1024]: every request against the oracle's union attention and its
    level-1 (+) level-2 fold."""
    b = I.shared_prefix_decode(seed=0)
    log(f"[composable plan] groups={b.groups} prefix={b.prefix_len} suffix {b.suffix_lens.min()}..{b.suffix_lens.max()}")
    q, k, v = b.torch_values("cuda")
    levels = [dict(kv_indptr=b.l1_kv_indptr, kv_indices=b.l1_kv_indices, last_page_len=b.l1_last_page_len,
                   qo_indptr=b.l1_qo_indptr),
              dict(kv_indptr=b.l2_kv_indptr, kv_indices=b.l2_kv_indices, last_page_len=b.l2_last_page_len)]
    p, o, l = _run_composable(levels, b, q, k, v)
    log(f"    plan: {p.export()['num_slots']} chunks")
    sm = 1.0 / math.sqrt(128)
    ro, rl, _, _ = A.composable_attention(
        b.q_f32, b.k_f32, b.v_f32, (b.l1_qo_indptr, b.l1_kv_indptr, b.l1_kv_indices, b.l1_last_page_len),
        (b.l2_kv_indptr, b.l2_kv_indices, b.l2_last_page_len), b.page_size, 32, 8, sm)
    compare(o, l, ro, rl, "bf16", "composable plan vs level fold")
    uo, ul = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.full_kv_indptr, b.full_kv_indices,
                               b.full_last_page_len, b.page_size, 32, 8, sm)
    compare(o, l, uo, ul, "bf16", "composable plan vs union")


def test_cascade_three_levels_one_plan():
    """A prompt shared by all 64 requests, 16 group prefixes of 4, private suffixes: three views in
    one composable plan, against the union attention."""
    b = I.cascade_decode(seed=0)
    log(f"[cascade plan] groups={b.groups} prefixes={b.prefix_lens}")
    q, k, v = b.torch_values("cuda")
    levels = [dict(kv_indptr=ip, kv_indices=ix, last_page_len=la, qo_indptr=qo) for qo, ip, ix, la in b.levels]
    ip, ix, la = b.suffix
    levels.append(dict(kv_indptr=ip, kv_indices=ix, last_page_len=la))
    _, o, l = _run_composable(levels, b, q, k, v)
    uo, ul = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, *b.full, b.page_size, 32, 8, 1.0 / math.sqrt(128))
    compare(o, l, uo, ul, "bf16", "cascade plan vs union")


def test_composable_with_empty_rows_and_few_workers():
    """Levels where some queries see no keys in one view (and one query in none), g = 2, 3 workers."""
    import torch

    nq = 9
    P = 4
    l1_kv, l1_qo = [37, 0, 90], [4, 2, 3]
    l2_kv = [5, 0, 17, 0, 0, 64, 0, 3, 29]
    rng = np.random.default_rng(3)
    lens = np.array(l1_kv + l2_kv)
    need = int(((lens + P - 1) // P).sum())
    perm = rng.permutation(need + 5)
    ip1, ix1, la1 = I.page_table_from_lengths(l1_kv, P, perm[:int(((np.array(l1_kv) + P - 1) // P).sum())])
    ip2, ix2, la2 = I.page_table_from_lengths(l2_kv, P, perm[len(ix1):])
    pool = need + 5
    Hq, Hk, d = 4, 2, 64
    q = torch.randn(nq, Hq, d, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    k = torch.randn(pool, P, Hk, d, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    v = torch.randn(pool, P, Hk, d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    from block_sparse_paged_bsr_amd import api

    qo1 = np.concatenate([[0], np.cumsum(l1_qo)]).astype(np.int32)
    p = api.ComposablePlan([dict(kv_indptr=ip1, kv_indices=ix1, last_page_len=la1, qo_indptr=qo1),
                            dict(kv_indptr=ip2, kv_indices=ix2, last_page_len=la2)],
                           num_pages=pool, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=d, page_size=P, num_workers=3)
    ws = api.alloc_workspace(p)
    p.upload(ws)
    o, l = api.run_prefill(p, ws, q.cuda(), k.cuda(), v.cuda(), sm_scale=0.3)
    torch.cuda.synchronize()
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
    ro, rl, _, _ = A.composable_attention(qf, kf, vf, (qo1, ip1, ix1, la1), (ip2, ix2, la2), P, Hq, Hk, 0.3)
    log("[composable small] 9 queries, empty rows")
    compare(o.float().cpu().numpy(), l.cpu().numpy(), ro, rl, "bf16", "composable with empty rows")
    # query 4: level 1's request 1 (queries 4-5) has no keys and its own suffix is empty
    assert np.isneginf(rl[4]).all() and np.isneginf(l.cpu().numpy()[4]).all()


@pytest.mark.parametrize("case", range(4))
def test_decode_kernel_on_multi_query_tiles(case):
    """Ordinary non-causal plans whose 16-row tiles hold several queries run on the decode kernel."""
    kv, qo, P, Hq, Hk, d, C_, cap = [
        ([300, 17, 64, 129], [5, 3, 16, 1], 16, 8, 2, 128, 7, 0.0),
        ([200, 50], [7, 11], 4, 16, 8, 64, 5, 0.0),
        ([1000], [2], 16, 32, 2, 128, 9, 0.0),
        ([300, 17, 64, 129], [5, 3, 16, 1], 16, 32, 8, 128, 11, 2.5),
    ][case]
    b = I.make_paged_batch(300 + case, kv, qo, page_size=P, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=d,
                           num_pages=sum((x + P - 1) // P for x in kv) + 3)
    log(f"[multi-query tiles] kv={kv} qo={qo} H={Hq}/{Hk} d={d} C={C_} cap={cap}")
    p = make_plan(b, num_workers=C_, tile_q=16, causal=False, soft_cap=cap)
    o, l, _ = run_gpu(b, p, decode=False)
    ro, rl = oracle(b, causal=False, soft_cap=cap)
    compare(o, l, ro, rl, "bf16", "multi-query tiles on the decode kernel")
