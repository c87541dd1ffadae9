"""GPU tests of the split-request fold inside the decode kernel: the wave that writes the
last partial state of a split request folds that request's states in the plan's slot order
("FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for LLM Inference Serving"
§VIII.3 and §VIII.6), so a decode call is one launch unless a request has no keys.

* Launch structure: the batch-64 decode (55 split requests, none empty) makes one attention launch
  and no merge launch per call; a batch with an empty request adds the merge launch, which then
  writes only the empty state.
* Determinism: repeated calls give bitwise-equal outputs, and the arrival counters return to zero
  (a second plan sharing nothing with the first still folds correctly after it).
* Parity against the fp64 oracle on batches with many splits per request (one worker per few
  hundred tokens), on every request.

Tolerances: bf16 inputs with fp32 accumulation -> O max-abs 2e-2, LSE max-abs 1e-2.
"""
import math

import numpy as np
import pytest

import workloads as I
from tests.gpu_helpers import compare, log, make_plan, oracle, run_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_paged_bsr_amd import api

    api.version()  # loads the library or raises


def _launches(p, b, calls=3):
    import torch
    from block_sparse_paged_bsr_amd import api

    q, k, v = b.torch_values("cuda")
    ws = api.alloc_workspace(p)
    p.upload(ws)
    outs = []
    api.timing_enable(True)
    try:
        for _ in range(calls):
            o, lse = api.run_decode(p, ws, q, k, v, sm_scale=1.0 / math.sqrt(b.head_dim))
            torch.cuda.synchronize()
            outs.append((o.float().cpu().numpy(), lse.cpu().numpy()))
        t = api.timing_read()
    finally:
        api.timing_enable(False)
    return t, outs


def test_batch64_decode_is_one_launch_and_deterministic():
    from block_sparse_paged_bsr_amd import api

    b = I.batched_decode_bf16(seed=0, poison=True)
    C_ = api.query_num_workers("decode", 32, 8, 128)
    p = make_plan(b, num_workers=C_)
    e = p.export()
    split = int(sum(1 for k in range(len(e["merge_ptr"]) - 1) if e["merge_ptr"][k + 1] > e["merge_ptr"][k]))
    log(f"[fold batch64] workers={C_} items={e['items'].shape[0]} split requests={split}")
    assert split > 0 and split == len(e["merge_ptr"]) - 1  # split requests only, none empty
    t, outs = _launches(p, b)
    assert t["attn_launches"] == 3 and t["merge_launches"] == 0, t
    for o, l in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(l, outs[0][1])
    reqs = list(range(0, 64, 8))
    ro, rl = oracle(b, requests=reqs)
    compare(outs[0][0], outs[0][1], ro, rl, "bf16", "batch-64 decode, folded in the kernel (8 requests)")


def test_empty_request_adds_the_merge_launch():
    b = I.make_paged_batch(21, [300, 0, 517, 64, 0, 1000], None, page_size=16, num_qo_heads=16, num_kv_heads=4,
                           head_dim=128, poison=True)
    p = make_plan(b, num_workers=7)
    log("[fold + empty] lens [300, 0, 517, 64, 0, 1000], 7 workers")
    t, outs = _launches(p, b, calls=2)
    assert t["attn_launches"] == 2 and t["merge_launches"] == 2, t
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    ro, rl = oracle(b)
    compare(outs[1][0], outs[1][1], ro, rl, "bf16", "fold + empty requests")


@pytest.mark.parametrize("seed,workers", [(31, 40), (32, 97), (33, 256)])
def test_many_splits_per_request(seed, workers):
    """Up to dozens of partial states per request, so the fold runs several rounds of eight slots,
    and counters of one plan are reused by the next call of another plan."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 3000, size=12)
    g = int(rng.choice([1, 2, 4, 8]))
    b = I.make_paged_batch(seed, lens, None, page_size=int(rng.choice([1, 8, 16])), num_qo_heads=4 * g,
                           num_kv_heads=4, head_dim=int(rng.choice([64, 128])), poison=True)
    p = make_plan(b, num_workers=workers)
    e = p.export()
    counts = np.diff(np.asarray(e["merge_ptr"]))
    log(f"[fold many splits] seed={seed} g={g} P={b.page_size} d={b.head_dim} workers={workers} "
        f"slots per split request up to {int(counts.max()) if counts.size else 0}")
    o, l, _ = run_gpu(b, p)
    o2, l2, _ = run_gpu(b, p)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    ro, rl = oracle(b)
    compare(o, l, ro, rl, "bf16", f"many splits (seed {seed})")
