"""GPU parity of the shared-prefix comparison of "FlashInfer: Making Attention Fit the Serving
Workload" §7.3 (Appendix Table 5 shapes: batch 64 with a 32,768-token prefix, batch 16 with a
1,024-token prefix, 128-token suffixes), in the launch configuration bench.py times: the prefix
view (one block row of all queries, non-causal, chunks of >= 256 keys), the suffix view (decode),
their merge, the two views as one composable plan, and the single-level view, against the fp64
oracle.  Batch 16 is compared on every
row; batch 64 on every fourth request, 16 of them (the oracle evaluates them one by one).

Tolerances: bf16 inputs with fp32 accumulation -> O max-abs 2e-2, LSE max-abs 1e-2.
"""
import math

import numpy as np
import pytest

import workloads as I
from oracle import attention as A
from tests.gpu_helpers import compare, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_paged_bsr_amd import api

    api.version()  # loads the library or raises


@pytest.mark.parametrize("R,P", [(16, 1024), (64, 32768)])
def test_shared_prefix_table5_shapes(R, P):
    import torch
    from block_sparse_paged_bsr_amd import api

    b = I.cascade_decode(seed=0, requests=R, groups=(1,), prefix_lens=(P,), suffix_lo=128, suffix_hi=128,
                         poison=True)
    log(f"[shared prefix] batch {R}, prefix {P}, suffix 128, pool {b.num_pages} pages")
    q, k, v = b.torch_values("cuda")
    sm = 1.0 / math.sqrt(b.head_dim)
    qo, ip, ix, la = b.levels[0]
    C1 = api.query_num_workers("prefill", 32, 8, 128)
    C2 = api.query_num_workers("decode", 32, 8, 128)
    mk = lambda C: api.Plan(ip, ix, la, num_pages=b.num_pages, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                            page_size=b.page_size, qo_indptr=qo, causal=False, num_workers=C)
    W = int(mk(C1).export()["total_work"])
    p1 = mk(max(1, min(C1, (W + 255) // 256)))
    sip, six, sla = b.suffix
    p2 = api.Plan(sip, six, sla, num_pages=b.num_pages, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                  page_size=b.page_size, num_workers=C2)
    pf = api.Plan(*b.full, num_pages=b.num_pages, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                  page_size=b.page_size, num_workers=C2)
    log(f"    prefix plan: {p1.export()['num_workers']} workers, {p1.export()['num_slots']} partial slots")
    states = []
    for p, fn in ((p1, api.run_prefill), (p2, api.run_decode), (pf, api.run_decode)):
        w = api.alloc_workspace(p)
        p.upload(w)
        states.append(fn(p, w, q, k, v, sm_scale=sm))
    o, l = api.merge_state(*states[0], *states[1])
    torch.cuda.synchronize()

    reqs = list(range(R)) if R <= 16 else list(range(0, R, 4))  # batch 64: every fourth request
    # prefix view: request 0 holds all R queries; check the queries of the sampled requests
    ro1, rl1 = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, ip, ix, la, b.page_size, 32, 8, sm, qo_indptr=qo,
                                 causal=False, query_subset={0: np.asarray(reqs)})
    ro2, rl2 = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, sip, six, sla, b.page_size, 32, 8, sm, requests=reqs)
    ruo, rul = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, *b.full, b.page_size, 32, 8, sm, requests=reqs)
    cpu = lambda st: (st[0].float().cpu().numpy(), st[1].cpu().numpy())
    compare(*cpu(states[0]), ro1, rl1, "bf16", "prefix view")
    compare(*cpu(states[1]), ro2, rl2, "bf16", "suffix view")
    compare(*cpu(states[2]), ruo, rul, "bf16", "single-level view")
    compare(*cpu((o, l)), ruo, rul, "bf16", "prefix (+) suffix vs union")

    # the same two views as one composable plan (one attention and one merge launch)
    cp = api.ComposablePlan([dict(kv_indptr=ip, kv_indices=ix, last_page_len=la, qo_indptr=qo),
                             dict(kv_indptr=sip, kv_indices=six, last_page_len=sla)],
                            num_pages=b.num_pages, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                            page_size=b.page_size, num_workers=C2)
    wc = api.alloc_workspace(cp)
    cp.upload(wc)
    log(f"    composable plan: {cp.export()['num_slots']} partial slots")
    oc, lc = api.run_prefill(cp, wc, q, k, v, sm_scale=sm)
    torch.cuda.synchronize()
    compare(*cpu((oc, lc)), ruo, rul, "bf16", "composable plan vs union")
