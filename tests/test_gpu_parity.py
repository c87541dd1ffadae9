"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances: bf16 inputs with fp32 accumulation -> O max-abs 2e-2, LSE max-abs 1e-2;
fp32 -> 1e-5 for both.  Plans and gathered row ids are compared bit for bit.
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


@pytest.mark.parametrize("num_workers", [1, 3, 8])
def test_tiny_decode_fp32(num_workers):
    log(f"[tiny_decode_fp32] workers={num_workers}")
    b = I.tiny_decode_fp32(seed=0)
    p = make_plan(b, num_workers=num_workers)
    o, l, _ = run_gpu(b, p)
    ro, rl = oracle(b)
    compare(o, l, ro, rl, "f32", "tiny fp32")


def test_gather_rows_bit_exact():
    import torch
    from block_sparse_paged_bsr_amd import api

    for b in (I.tiny_decode_fp32(0), I.make_paged_batch(3, [1, 17, 0, 64, 5], None, page_size=16,
                                                         num_qo_heads=4, num_kv_heads=2, head_dim=64,
                                                         num_pages=40)):
        log(f"[gather_rows] {b.name} lens={b.kv_lens.tolist()}")
        p = make_plan(b, num_workers=4)
        ws = api.alloc_workspace(p)
        p.upload(ws)
        total = int(b.kv_lens.sum())
        rows = api.debug_gather_rows(p, ws, total).cpu().numpy()
        torch.cuda.synchronize()
        ref = np.concatenate([A.physical_rows(b.kv_indptr, b.kv_indices, b.last_page_len, b.page_size, i)
                              for i in range(b.batch)])
        assert np.array_equal(rows, ref)


DECODE_CASES = [
    # (lens, P, Hq, Hk, d, workers)
    ([37, 1, 200, 16, 513], 16, 32, 8, 128, 8),
    ([37, 1, 200, 16, 513], 16, 32, 8, 128, 1),
    ([100, 0, 260, 31], 4, 8, 8, 128, 5),
    ([333, 70, 1], 1, 16, 4, 64, 6),
    ([129, 300], 16, 16, 2, 128, 7),  # g = 8: two waves per KV head
    ([129, 300], 16, 6, 2, 128, 7),   # g = 3: served by the tiled kernel
]


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_decode_bf16_small(case):
    lens, P, Hq, Hk, d, C_ = DECODE_CASES[case]
    log(f"[decode_bf16_small] lens={lens} P={P} H={Hq}/{Hk} d={d} workers={C_}")
    b = I.make_paged_batch(case, lens, None, page_size=P, num_qo_heads=Hq, num_kv_heads=Hk,
                           head_dim=d, num_pages=sum((x + P - 1) // P for x in lens) + 7)
    p = make_plan(b, num_workers=C_)
    o, l, _ = run_gpu(b, p)
    ro, rl = oracle(b)
    compare(o, l, ro, rl, "bf16", "decode small")


def test_decode_bf16_batch64_full():
    """Batch-64 paged decode at its full size: every request against the oracle."""
    import torch
    from block_sparse_paged_bsr_amd import api

    b = I.batched_decode_bf16(seed=0)
    C_ = api.query_num_workers("decode", 32, 8, 128)
    log(f"[decode_bf16_batch64_full] tokens={int(b.kv_lens.sum())} workers={C_}")
    p = make_plan(b, num_workers=C_)
    tens = b.torch_values("cuda")
    o, l, ws = run_gpu(b, p, tensors=tens)
    ro, rl = oracle(b)
    compare(o, l, ro, rl, "bf16", "decode batch64")
    # run twice: bitwise identical (fixed plan, no atomics)
    o2, l2, _ = run_gpu(b, p, tensors=tens)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    torch.cuda.synchronize()


PREFILL_CASES = [
    # (kv lens, qo lens, P, Hq, Hk, d, causal, workers, tile_q)
    ([300, 17, 64, 129], [300, 17, 64, 129], 16, 8, 2, 128, True, 9, 0),
    ([300, 17, 64, 129], [300, 17, 64, 129], 16, 8, 2, 128, False, 3, 0),
    ([500, 40], [7, 40], 4, 8, 8, 64, True, 5, 0),        # l_qo < l_kv: bottom-right
    ([20, 100], [50, 3], 16, 4, 1, 128, True, 4, 16),     # l_qo > l_kv: empty rows
    ([250, 90], [250, 90], 1, 12, 4, 128, True, 11, 32),  # page size 1, g = 3
    ([64, 0, 33], [16, 5, 9], 16, 16, 4, 128, False, 2, 64),  # empty request
    ([700, 260, 1031], [700, 200, 1031], 16, 32, 8, 64, True, 30, 128),  # 128-row shape, d = 64
    ([700, 260], [700, 260], 8, 16, 4, 128, True, 40, 128),   # 128-row shape, page size 8
    ([700, 260], [700, 260], 12, 16, 4, 128, True, 40, 128),  # 128-row shape, page size 12
]


@pytest.mark.parametrize("case", range(len(PREFILL_CASES)))
def test_prefill_bf16_small(case):
    kv, qo, P, Hq, Hk, d, causal, C_, tq = PREFILL_CASES[case]
    log(f"[prefill_bf16_small] kv={kv} qo={qo} P={P} H={Hq}/{Hk} d={d} causal={causal} C={C_} Tq={tq}")
    b = I.make_paged_batch(100 + case, kv, qo, page_size=P, num_qo_heads=Hq, num_kv_heads=Hk,
                           head_dim=d, causal=causal, num_pages=sum((x + P - 1) // P for x in kv) + 5)
    p = make_plan(b, num_workers=C_, tile_q=tq)
    o, l, _ = run_gpu(b, p)
    ro, rl = oracle(b)
    compare(o, l, ro, rl, "bf16", "prefill small")


def test_prefill_bf16_ragged_full_sampled():
    """Ragged causal prefill at full size (batch 16, lengths U[256, 4096]); sampled rows."""
    from block_sparse_paged_bsr_amd import api

    b = I.ragged_prefill_bf16(seed=0)
    C_ = api.query_num_workers("prefill", 32, 8, 128)
    log(f"[prefill_bf16_ragged_full] lens={b.kv_lens.tolist()} workers={C_}")
    p = make_plan(b, num_workers=C_)
    o, l, _ = run_gpu(b, p)
    rng = np.random.default_rng(0)
    sub = {i: np.unique(np.concatenate([[0, 1, int(b.qo_lens[i]) - 1],
                                        rng.integers(0, int(b.qo_lens[i]), 24)])) for i in range(b.batch)}
    ro, rl = oracle(b, query_subset=sub)
    compare(o, l, ro, rl, "bf16", "prefill ragged full (sampled rows)")


def test_merge_state_kernel():
    import torch
    from block_sparse_paged_bsr_amd import api

    rng = np.random.default_rng(0)
    R, H, d = 37, 5, 128
    for dt, tol in ((torch.float32, 1e-6), (torch.bfloat16, 1e-2)):
        oa = torch.from_numpy(rng.standard_normal((R, H, d)).astype(np.float32)).to(dt)
        ob = torch.from_numpy(rng.standard_normal((R, H, d)).astype(np.float32)).to(dt)
        la = rng.standard_normal((R, H)).astype(np.float32) * 4
        lb = rng.standard_normal((R, H)).astype(np.float32) * 4
        la[0, :] = -np.inf
        lb[1, :] = -np.inf
        la[2, :] = -np.inf
        lb[2, :] = -np.inf
        oa[2] = 0
        ob[2] = 0
        ro, rl = A.merge_state(oa.float().numpy(), la, ob.float().numpy(), lb)
        ga, gb = oa.cuda(), ob.cuda()
        gla, glb = torch.from_numpy(la).cuda(), torch.from_numpy(lb).cuda()
        o, l = api.merge_state(ga, gla, gb, glb)
        torch.cuda.synchronize()
        o = o.float().cpu().numpy()
        l = l.cpu().numpy()
        assert np.array_equal(np.isneginf(l), np.isneginf(rl))
        fin = np.isfinite(rl)
        assert np.max(np.abs(l[fin] - rl[fin])) < 1e-5
        assert np.max(np.abs(o - ro)) < tol
        # in place: out aliases a
        o2, l2 = api.merge_state(ga, gla, gb, glb, o_out=ga, lse_out=gla)
        torch.cuda.synchronize()
        assert np.array_equal(o2.float().cpu().numpy(), o) and np.array_equal(l2.cpu().numpy(), l)


def test_composable_shared_prefix():
    """Two BSR levels (shared prefix at 4 queries per block row + private suffixes) + merge."""
    import torch
    from block_sparse_paged_bsr_amd import api

    b = I.shared_prefix_decode(seed=0)
    log(f"[composable] groups={b.groups} prefix={b.prefix_len} suffix={b.suffix_lens.min()}..{b.suffix_lens.max()}")
    q, k, v = b.torch_values("cuda")
    sm = 1.0 / math.sqrt(b.head_dim)
    C1 = api.query_num_workers("prefill", 32, 8, 128)
    C2 = api.query_num_workers("decode", 32, 8, 128)
    p1 = api.Plan(b.l1_kv_indptr, b.l1_kv_indices, b.l1_last_page_len, num_pages=b.num_pages,
                  num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=b.page_size,
                  qo_indptr=b.l1_qo_indptr, causal=False, num_workers=C1)
    p2 = api.Plan(b.l2_kv_indptr, b.l2_kv_indices, b.l2_last_page_len, num_pages=b.num_pages,
                  num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=b.page_size,
                  num_workers=C2)
    w1, w2 = api.alloc_workspace(p1), api.alloc_workspace(p2)
    p1.upload(w1)
    p2.upload(w2)
    o1, l1 = api.run_prefill(p1, w1, q, k, v, sm_scale=sm)
    o2, l2 = api.run_decode(p2, w2, q, k, v, sm_scale=sm)
    o, l = api.merge_state(o1, l1, o2, l2)
    torch.cuda.synchronize()
    ro, rl, (ro1, rl1), (ro2, rl2) = A.composable_attention(
        b.q_f32, b.k_f32, b.v_f32,
        (b.l1_qo_indptr, b.l1_kv_indptr, b.l1_kv_indices, b.l1_last_page_len),
        (b.l2_kv_indptr, b.l2_kv_indices, b.l2_last_page_len), b.page_size, 32, 8, sm)
    compare(o1.float().cpu().numpy(), l1.cpu().numpy(), ro1, rl1, "bf16", "composable level 1")
    compare(o2.float().cpu().numpy(), l2.cpu().numpy(), ro2, rl2, "bf16", "composable level 2")
    compare(o.float().cpu().numpy(), l.cpu().numpy(), ro, rl, "bf16", "composable merged")


def test_cascade_three_levels():
    """Multi-level cascade: a prompt shared by all 64 requests, group prefixes (16 x 4) and
    private suffixes, as three BSR views merged left to right with merge_state."""
    import torch
    from block_sparse_paged_bsr_amd import api

    b = I.cascade_decode(seed=0)
    log(f"[cascade] groups={b.groups} prefixes={b.prefix_lens} suffix={b.suffix_lens.min()}..{b.suffix_lens.max()}")
    q, k, v = b.torch_values("cuda")
    sm = 1.0 / math.sqrt(b.head_dim)
    C1 = api.query_num_workers("prefill", 32, 8, 128)
    C2 = api.query_num_workers("decode", 32, 8, 128)
    states = []
    for qo, ip, ix, la in b.levels:
        p = api.Plan(ip, ix, la, num_pages=b.num_pages, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                     page_size=b.page_size, qo_indptr=qo, causal=False, num_workers=C1)
        w = api.alloc_workspace(p)
        p.upload(w)
        states.append(api.run_prefill(p, w, q, k, v, sm_scale=sm))
    ip, ix, la = b.suffix
    p = api.Plan(ip, ix, la, num_pages=b.num_pages, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                 page_size=b.page_size, num_workers=C2)
    w = api.alloc_workspace(p)
    p.upload(w)
    states.append(api.run_decode(p, w, q, k, v, sm_scale=sm))
    o, l = states[0]
    for o2, l2 in states[1:]:
        o, l = api.merge_state(o, l, o2, l2)
    torch.cuda.synchronize()
    ro, rl, rstates = A.cascade_attention(b.q_f32, b.k_f32, b.v_f32, b.levels, b.suffix, b.page_size, 32, 8, sm)
    for i, ((og, lg), (orf, lrf)) in enumerate(zip(states, rstates)):
        compare(og.float().cpu().numpy(), lg.cpu().numpy(), orf, lrf, "bf16", f"cascade view {i}")
    compare(o.float().cpu().numpy(), l.cpu().numpy(), ro, rl, "bf16", "cascade merged")
    uo, ul = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, *b.full, b.page_size, 32, 8, sm)
    compare(o.float().cpu().numpy(), l.cpu().numpy(), uo, ul, "bf16", "cascade vs union")


def test_cascade_levels_on_separate_streams():
    """The cascade's levels run on three streams joined before the fold: bitwise equal to the
    same calls in sequence (each level's plan and workspace are its own)."""
    import torch
    from block_sparse_paged_bsr_amd import api

    b = I.cascade_decode(seed=1)
    log("[cascade_streams] three levels on three streams")
    q, k, v = b.torch_values("cuda")
    sm = 1.0 / math.sqrt(b.head_dim)
    runs = []
    for qo, ip, ix, la in b.levels:
        p = api.Plan(ip, ix, la, num_pages=b.num_pages, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                     page_size=b.page_size, qo_indptr=qo, causal=False, num_workers=64)
        runs.append((p, api.run_prefill))
    ip, ix, la = b.suffix
    runs.append((api.Plan(ip, ix, la, num_pages=b.num_pages, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                          page_size=b.page_size, num_workers=128), api.run_decode))
    wss = []
    for p, _ in runs:
        w = api.alloc_workspace(p)
        p.upload(w)
        wss.append(w)
    torch.cuda.synchronize()

    def fold(states):
        o, l = states[0]
        for o2, l2 in states[1:]:
            o, l = api.merge_state(o, l, o2, l2)
        return o, l

    seq = fold([fn(p, w, q, k, v, sm_scale=sm) for (p, fn), w in zip(runs, wss)])
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in runs]
    cur = torch.cuda.current_stream()
    outs = []
    for st, (p, fn), w in zip(streams, runs, wss):
        st.wait_stream(cur)
        with torch.cuda.stream(st):
            outs.append(fn(p, w, q, k, v, sm_scale=sm))
    for st in streams:
        cur.wait_stream(st)
    par = fold(outs)
    torch.cuda.synchronize()
    assert torch.equal(seq[0], par[0]) and torch.equal(seq[1], par[1])


@pytest.mark.parametrize("br,bc", [(16, 16), (64, 16), (4, 32), (128, 64)])
def test_block_sparse_attention_bsr(br, bc):
    """Block-sparse attention of one 1024-token sequence, as a BSR matrix of B_r x B_c blocks
    (35 % present): block rows are the plan's requests, column blocks its pages; against
    the oracle's dense attention under the expanded block mask."""
    bs = I.block_sparse_attention(40 + br, 1024, br, bc, 0.35, num_qo_heads=32, num_kv_heads=8, head_dim=128)
    b = bs.dense
    log(f"[block_sparse] L=1024 B_r={br} B_c={bc} blocks={int(bs.block_mask.sum())}/{bs.block_mask.size}")
    p = make_plan(b, num_workers=64, causal=False)
    o, l, _ = run_gpu(b, p, decode=False)
    dense_mask = np.kron(bs.block_mask, np.ones((br, bc), dtype=bool))
    npg = b.k_f32.shape[0]
    ro, rl = A.batch_attention(b.q_f32, b.k_f32, b.v_f32, [0, npg], np.arange(npg), [bc], bc, 32, 8,
                               1.0 / math.sqrt(128), qo_indptr=[0, 1024], custom_mask=[dense_mask])
    compare(o, l, ro, rl, "bf16", f"block sparse {br}x{bc}")
