"""GPU: the run calls captured in a HIP graph and replayed (plan once, replay per step).

The plan's metadata is uploaded before capture; a run launches only kernels on the
caller's stream (no allocation, no memset, no host synchronisation), so it can be
captured.  Each replay is compared bit for bit with an eager run on the same inputs,
with eager work and synchronisations between the replays, and the replayed result is
checked against the fp64 oracle.
"""
import math

import numpy as np
import pytest

import workloads as I
from tests.gpu_helpers import compare, log, make_plan, oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_paged_bsr_amd import api

    api.version()


def _graph_case(b, kind, num_workers):
    import torch
    from block_sparse_paged_bsr_amd import api

    p = make_plan(b, num_workers=num_workers)
    ws = api.alloc_workspace(p)
    p.upload(ws)
    torch.cuda.synchronize()
    q, k, v = b.torch_values("cuda")
    fn = api.run_decode if kind == "decode" else api.run_prefill
    sm = 1.0 / math.sqrt(b.head_dim)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], b.num_qo_heads, dtype=torch.float32, device="cuda")
    # warm up on a side stream (graph capture requirement), then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(p, ws, q, k, v, o=o, lse=lse, sm_scale=sm)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(p, ws, q, k, v, o=o, lse=lse, sm_scale=sm)
    torch.cuda.synchronize()
    q0 = q.clone()
    for rep in range(3):
        # new query values in place, then the replay and an eager run on the same inputs
        q.copy_(q0 * (1.0 + 0.25 * rep))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        og, lg = o.clone(), lse.clone()
        oe, le = fn(p, ws, q, k, v, sm_scale=sm)
        torch.cuda.synchronize()
        assert torch.equal(og, oe) and torch.equal(lg, le), f"replay {rep} differs from the eager run"
        log(f"    replay {rep}: bitwise equal to the eager run")
    return og.float().cpu().numpy(), lg.cpu().numpy(), q


def test_graph_replay_decode():
    b = I.make_paged_batch(11, [37, 1, 200, 16, 513, 0, 129], None, page_size=16, num_qo_heads=32,
                           num_kv_heads=8, head_dim=128)
    log(f"[graph_decode] lens={b.kv_lens.tolist()}")
    o, l, q = _graph_case(b, "decode", num_workers=8)
    # the last replay ran with q * 1.5: the oracle on those inputs
    b.q_f32 = q.float().cpu().numpy()
    ro, rl = oracle(b)
    compare(o, l, ro, rl, "bf16", "graph-replayed decode")


def test_graph_replay_prefill():
    b = I.make_paged_batch(12, [300, 17, 64, 129], [300, 17, 64, 129], page_size=16, num_qo_heads=8,
                           num_kv_heads=2, head_dim=128, causal=True)
    log(f"[graph_prefill] lens={b.kv_lens.tolist()}")
    o, l, q = _graph_case(b, "prefill", num_workers=9)
    b.q_f32 = q.float().cpu().numpy()
    ro, rl = oracle(b)
    compare(o, l, ro, rl, "bf16", "graph-replayed prefill")
