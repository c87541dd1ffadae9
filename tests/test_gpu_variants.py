"""GPU parity of the attention variants against the oracle: sliding window and logits soft cap.

The window ("FlashInfer 原理" §⑧) is applied by the planner (each tile's KV range starts at
its first row's window) and by a per-row lower bound in the prefill kernels; the soft cap
("FlashInfer: Making Attention Fit the Serving Workload" §5, eq. 8) transforms every score
before the mask.  Caps of a few units make tanh saturate on part of the scores, so a wrong
transform cannot hide.  Same tolerances as the plain path.
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


DECODE_VAR = [
    # (lens, P, Hq, Hk, d, workers, window_left, soft_cap)
    ([37, 1, 200, 16, 513], 16, 32, 8, 128, 8, 100, 0.0),
    ([37, 1, 200, 16, 513], 16, 32, 8, 128, 8, -1, 2.0),
    ([37, 1, 200, 16, 513], 16, 32, 8, 128, 3, 0, 5.0),      # window 0: the last key only
    ([333, 70, 1, 900], 1, 16, 4, 64, 6, 63, 1.5),
    ([129, 300], 16, 6, 2, 128, 7, 200, 3.0),                 # g = 3: the tiled kernel
]


@pytest.mark.parametrize("case", range(len(DECODE_VAR)))
def test_decode_variants_bf16(case):
    lens, P, Hq, Hk, d, C_, w, cap = DECODE_VAR[case]
    log(f"[decode_variants_bf16] lens={lens} P={P} H={Hq}/{Hk} d={d} C={C_} window={w} cap={cap}")
    b = I.make_paged_batch(300 + case, lens, None, page_size=P, num_qo_heads=Hq, num_kv_heads=Hk,
                           head_dim=d, num_pages=sum((x + P - 1) // P for x in lens) + 3)
    p = make_plan(b, num_workers=C_, window_left=w, soft_cap=cap)
    o, l, _ = run_gpu(b, p)
    ro, rl = oracle(b, window_left=w, soft_cap=cap)
    compare(o, l, ro, rl, "bf16", "decode variant")


PREFILL_VAR = [
    # (kv lens, qo lens, P, Hq, Hk, d, causal, workers, tile_q, window_left, soft_cap)
    ([300, 17, 64, 129], [300, 17, 64, 129], 16, 8, 2, 128, True, 60, 0, 40, 0.0),
    ([300, 17, 64, 129], [300, 17, 64, 129], 16, 8, 2, 128, True, 40, 0, -1, 2.5),
    ([300, 17, 64, 129], [300, 17, 64, 129], 16, 8, 2, 128, False, 3, 0, 70, 4.0),
    ([500, 40], [7, 40], 4, 8, 8, 64, True, 5, 0, 0, 0.0),          # diagonal only
    ([700, 260], [700, 260], 16, 32, 8, 128, True, 100, 128, 100, 3.0),  # 128-row tiles, capped
    ([700, 260], [700, 260], 16, 32, 8, 128, True, 100, 128, 100, 0.0),  # 128-row shape, window
    ([700, 260], [700, 260], 16, 32, 8, 128, True, 13, 64, 333, 0.0),   # 64-row tiles
    ([250, 90], [250, 90], 1, 12, 4, 128, True, 11, 32, 31, 1.5),       # page size 1, g = 3
    ([20, 100], [50, 3], 16, 4, 1, 128, True, 4, 16, 5, 2.0),           # l_qo > l_kv: empty rows
    ([1200], [1200], 12, 8, 1, 128, True, 150, 0, 257, 0.0),            # page size 12 (no power of two)
]


@pytest.mark.parametrize("case", range(len(PREFILL_VAR)))
def test_prefill_variants_bf16(case):
    kv, qo, P, Hq, Hk, d, causal, C_, tq, w, cap = PREFILL_VAR[case]
    log(f"[prefill_variants_bf16] kv={kv} qo={qo} P={P} H={Hq}/{Hk} d={d} causal={causal} C={C_} "
        f"Tq={tq} window={w} cap={cap}")
    b = I.make_paged_batch(400 + case, kv, qo, page_size=P, num_qo_heads=Hq, num_kv_heads=Hk,
                           head_dim=d, causal=causal, num_pages=sum((x + P - 1) // P for x in kv) + 5)
    p = make_plan(b, num_workers=C_, tile_q=tq, window_left=w, soft_cap=cap)
    o, l, _ = run_gpu(b, p)
    ro, rl = oracle(b, window_left=w, soft_cap=cap)
    compare(o, l, ro, rl, "bf16", "prefill variant")


@pytest.mark.parametrize("decode", [True, False])
def test_variants_fp32(decode):
    log(f"[variants_fp32] decode={decode}")
    kv = [90, 1, 333, 47]
    qo = None if decode else [30, 1, 100, 47]
    b = I.make_paged_batch(500 + int(decode), kv, qo, page_size=8, num_qo_heads=8, num_kv_heads=2,
                           head_dim=64, dtype="f32", causal=not decode)
    p = make_plan(b, num_workers=5, window_left=20, soft_cap=2.0)
    o, l, _ = run_gpu(b, p)
    ro, rl = oracle(b, window_left=20, soft_cap=2.0)
    compare(o, l, ro, rl, "f32", "fp32 variant")


@pytest.mark.parametrize("cap", [5.0, 0.0])
def test_prefill_variants_ragged_full_sampled(cap):
    """Ragged causal prefill at full size (batch 16, lengths U[256, 4096]) with a 1024-key
    window, with and without a soft cap of 5; sampled rows of every request against the
    oracle."""
    from block_sparse_paged_bsr_amd import api

    b = I.ragged_prefill_bf16(seed=0)
    C_ = api.query_num_workers("prefill", 32, 8, 128)
    w = 1024
    log(f"[prefill_variants_ragged_full] lens={b.kv_lens.tolist()} workers={C_} window={w} cap={cap}")
    p = make_plan(b, num_workers=C_, window_left=w, soft_cap=cap)
    o, l, _ = run_gpu(b, p)
    rng = np.random.default_rng(1)
    sub = {i: np.unique(np.concatenate([[0, 1, int(b.qo_lens[i]) - 1],
                                        rng.integers(0, int(b.qo_lens[i]), 24)])) for i in range(b.batch)}
    ro, rl = oracle(b, query_subset=sub, window_left=w, soft_cap=cap)
    compare(o, l, ro, rl, "bf16", "prefill variant ragged full (sampled rows)")
