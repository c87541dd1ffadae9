"""GPU parity of the merge pass on tiles split into many partial slots: one 128-row query tile
(32 positions x 4 heads) over a long non-causal KV range, planned for so many workers that the
tile is cut into more than 256 chunks (the weights past the 256 kept in LDS are recomputed from
the LSEs) and into more than 1024 chunks (the slot list is read from memory instead of LDS).
Reduction map of "FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for LLM
Inference Serving" §VIII.5; the fold is eq. 6 of "FlashInfer: Making Attention Fit the Serving
Workload".  Tolerances: bf16 O max-abs 2e-2, LSE max-abs 1e-2.
"""
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


@pytest.mark.parametrize("kv_len,workers,min_slots", [(8192, 600, 300), (16384, 1300, 1100)])
def test_merge_many_slots(kv_len, workers, min_slots):
    b = I.make_paged_batch(3, np.array([kv_len]), np.array([32]), page_size=16, num_qo_heads=4, num_kv_heads=1,
                           head_dim=128)
    p = make_plan(b, num_workers=workers, tile_q=128, causal=False)
    ex = p.export()
    slots = int(ex["num_slots"])
    log(f"[merge] kv {kv_len}, {workers} workers: {slots} partial slots in {len(ex['merge_tiles'])} merge tile(s)")
    assert slots >= min_slots
    o, lse, _ = run_gpu(b, p, decode=False)
    ro, rl = oracle(b, causal=False)
    compare(o, lse, ro, rl, "bf16", f"{slots} slots")
