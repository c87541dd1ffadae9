"""GPU parity of custom masks (bsr_run_prefill_masked) against the oracle: random masks,
tree-shaped masks of speculative decoding (each draft token sees the prompt and its own
ancestors), masks combined with causal, window and soft cap, decode plans, fp32 and bf16,
rows left with no key."""
import math

import numpy as np
import pytest

import workloads as I
from oracle import attention as A
from tests.gpu_helpers import compare, log, make_plan

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_paged_bsr_amd import api

    api.version()  # loads the library or raises


def _run(b, p, masks):
    import torch
    from block_sparse_paged_bsr_amd import api

    q, k, v = b.torch_values("cuda")
    ws = api.alloc_workspace(p)
    p.upload(ws)
    bits = torch.from_numpy(api.pack_custom_mask(masks)).to("cuda")
    o, lse = api.run_prefill_masked(p, ws, q, k, v, bits, sm_scale=1.0 / math.sqrt(b.head_dim))
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _oracle(b, masks, window_left=-1, soft_cap=0.0):
    return A.batch_attention(b.q_f32, b.k_f32, b.v_f32, b.kv_indptr, b.kv_indices, b.last_page_len, b.page_size,
                             b.num_qo_heads, b.num_kv_heads, 1.0 / math.sqrt(b.head_dim), qo_indptr=b.qo_indptr,
                             causal=b.causal, window_left=window_left, soft_cap=soft_cap, custom_mask=masks)


def _random_masks(rng, qo, kv, density):
    return [rng.random((a, c)) < density for a, c in zip(qo, kv)]


def _tree_masks(rng, prompt, drafts):
    """Request i: prompt[i] tokens visible to every draft token, then drafts[i] draft tokens
    forming a random tree (parent of token t is a random earlier draft token or the prompt);
    a draft token sees the prompt, its ancestors and itself."""
    out = []
    for L, T in zip(prompt, drafts):
        m = np.zeros((T, L + T), dtype=bool)
        m[:, :L] = True
        parent = [-1] + [int(rng.integers(-1, t)) for t in range(1, T)]
        for t in range(T):
            a = t
            while a >= 0:
                m[t, L + a] = True
                a = parent[a]
        out.append(m)
    return out


CASES = [
    # (kv, qo, P, Hq, Hk, d, causal, workers, tile_q, dtype, density)
    ([300, 17, 64, 129], [40, 17, 64, 3], 16, 8, 2, 128, False, 9, 0, "bf16", 0.5),
    ([300, 17, 64, 129], [40, 17, 64, 3], 16, 8, 2, 128, True, 9, 0, "bf16", 0.7),
    ([700, 260], [300, 260], 16, 32, 8, 128, True, 40, 128, "bf16", 0.9),   # 128-row plans
    ([500, 40], [7, 40], 4, 8, 8, 64, False, 5, 32, "bf16", 0.3),
    ([250, 90], [250, 90], 1, 12, 4, 128, True, 11, 64, "bf16", 0.5),
    ([90, 1, 333], [30, 1, 100], 8, 8, 2, 64, True, 5, 0, "f32", 0.5),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_masks(case):
    kv, qo, P, Hq, Hk, d, causal, C_, tq, dt, dens = CASES[case]
    log(f"[masks] kv={kv} qo={qo} P={P} H={Hq}/{Hk} d={d} causal={causal} C={C_} Tq={tq} {dt} density={dens}")
    b = I.make_paged_batch(900 + case, kv, qo, page_size=P, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=d,
                           dtype=dt, causal=causal, num_pages=sum((x + P - 1) // P for x in kv) + 5)
    masks = _random_masks(np.random.default_rng(case), qo, kv, dens)
    masks[0][0, :] = False  # one row with no key at all
    p = make_plan(b, num_workers=C_, tile_q=tq)
    o, l = _run(b, p, masks)
    ro, rl = _oracle(b, masks)
    compare(o, l, ro, rl, dt, "custom mask")


def test_tree_masks_speculative_decoding():
    rng = np.random.default_rng(3)
    prompt, drafts = [500, 1200, 64], [16, 7, 31]
    kv = [a + t for a, t in zip(prompt, drafts)]
    log(f"[tree masks] prompt={prompt} drafts={drafts}")
    b = I.make_paged_batch(950, kv, drafts, page_size=16, num_qo_heads=32, num_kv_heads=8, head_dim=128)
    masks = _tree_masks(rng, prompt, drafts)
    p = make_plan(b, num_workers=24)
    o, l = _run(b, p, masks)
    ro, rl = _oracle(b, masks)
    compare(o, l, ro, rl, "bf16", "tree mask")


def test_mask_with_window_and_cap():
    kv, qo = [600, 333], [200, 100]
    log("[masks] with window 150 and soft cap 4")
    b = I.make_paged_batch(960, kv, qo, page_size=16, num_qo_heads=16, num_kv_heads=4, head_dim=128, causal=True)
    masks = _random_masks(np.random.default_rng(9), qo, kv, 0.6)
    p = make_plan(b, num_workers=20, window_left=150, soft_cap=4.0)
    o, l = _run(b, p, masks)
    ro, rl = _oracle(b, masks, window_left=150, soft_cap=4.0)
    compare(o, l, ro, rl, "bf16", "mask + window + cap")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_mask_on_a_decode_plan(dt):
    kv = [37, 1, 200, 16, 513]
    log(f"[masks] decode plan {dt}")
    b = I.make_paged_batch(970, kv, None, page_size=16, num_qo_heads=32, num_kv_heads=8,
                           head_dim=128 if dt == "bf16" else 64, dtype=dt, num_pages=60)
    masks = _random_masks(np.random.default_rng(4), [1] * len(kv), kv, 0.5)
    p = make_plan(b, num_workers=8)
    o, l = _run(b, p, masks)
    ro, rl = _oracle(b, masks)
    compare(o, l, ro, rl, dt, "decode plan + mask")


def test_missing_mask_is_rejected():
    import torch
    from block_sparse_paged_bsr_amd import _lib, api

    b = I.make_paged_batch(980, [40, 9], [4, 9], page_size=16, num_qo_heads=8, num_kv_heads=2, head_dim=128)
    p = make_plan(b, num_workers=4)
    ws = api.alloc_workspace(p)
    p.upload(ws)
    q, k, v = b.torch_values("cuda")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[0], 8, dtype=torch.float32, device="cuda")
    import ctypes as C
    rc = _lib.lib().bsr_run_prefill_masked(p.handle, C.c_void_p(ws.data_ptr()), C.c_void_p(q.data_ptr()),
                                           C.c_void_p(k.data_ptr()), C.c_void_p(v.data_ptr()), None,
                                           C.c_void_p(o.data_ptr()),
                                           C.cast(C.c_void_p(lse.data_ptr()), C.POINTER(C.c_float)), 1, 0.1, None)
    assert rc == _lib.BSR_INVALID_ARG
    short = torch.zeros(3, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        api.run_prefill_masked(p, ws, q, k, v, short)
    torch.cuda.synchronize()
