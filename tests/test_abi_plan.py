"""C-ABI checks that need no GPU: exports, host planner parity with the oracle, errors.

bsr_plan_create/export/destroy/workspace_bytes are pure host code, so they run here.
"""
import ctypes as C
import os
import re
import subprocess

import numpy as np
import pytest

from block_sparse_paged_bsr_amd import _lib
from block_sparse_paged_bsr_amd import api
import workloads as I
from oracle import plan as PL
from tests.conftest import ROOT, load_golden

HEADER = os.path.join(ROOT, "include", "bsr_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libbsr_attn.so not built")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|void|const char\*)\s+(bsr_\w+)\s*\(", src, re.M)))


def test_header_symbols_exported():
    names = _declared()
    assert len(names) >= 14
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\b(bsr_\w+)\b", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(_lib.EXPORTED) == names
    L = _lib.lib()
    for n in names:
        assert hasattr(L, n)
    assert "gfx950" in api.version()


def test_probe_header_symbols_exported():
    """include/bsr_probe.h against libbsr_probe.so (the HBM read and execution-rate probes
    bench.py uses): every declaration exported, arguments checked on the host before a launch."""
    if not os.path.exists(_lib.PROBE_PATH):
        pytest.skip("libbsr_probe.so not built")
    src = open(os.path.join(ROOT, "include", "bsr_probe.h")).read()
    names = sorted(set(re.findall(r"^\s*int\s+(bsr_\w+)\s*\(", src, re.M)))
    assert names == sorted(_lib.PROBE_EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.PROBE_PATH], capture_output=True, text=True).stdout
    assert set(names) <= set(re.findall(r"\b(bsr_\w+)\b", out))
    L = _lib.probe()
    # argument checks happen on the host, before any launch
    one = C.c_void_p(16)
    assert L.bsr_probe_read_pages(None, one, one, 1, 4096, 1, 0, one, None) == -1
    assert L.bsr_probe_read_pages(one, one, one, 1, 4000, 1, 0, one, None) == -1
    assert L.bsr_probe_read_pages(one, one, one, 1, 4096, 0, 0, one, None) == -1
    assert L.bsr_probe_read_pages(one, one, one, -1, 4096, 1, 0, one, None) == -1
    assert L.bsr_probe_read_pages(one, one, one, 0, 4096, 1, 0, one, None) == 0
    assert L.bsr_probe_issue_mix(-1, 1, one, one, None) == -1
    assert L.bsr_probe_issue_mix(8, 1, one, one, None) == -1
    assert L.bsr_probe_issue_mix(0, 0, one, one, None) == -1
    assert L.bsr_probe_issue_mix(0, 1, None, one, None) == -1
    assert L.bsr_probe_lds_read(2, 1, 1, one, one, None) == -1
    assert L.bsr_probe_lds_read(0, 5, 1, one, one, None) == -1
    assert L.bsr_probe_lds_read(0, 1, 1, one, None, None) == -1
    assert L.bsr_probe_l2_to_lds(None, 1, 1, 1, one, one, None) == -1
    assert L.bsr_probe_l2_to_lds(one, 0, 1, 1, one, one, None) == -1
    assert L.bsr_probe_l2_to_lds(one, 1, 0, 1, one, one, None) == -1


def _oracle_as_export(p):
    tiles = np.array([[t.req, t.row_start, t.row_end, t.vis, len(t.items)] for t in p.tiles], dtype=np.int32).reshape(-1, 5)
    items = np.array([[it.req, it.tile, it.row_start, it.row_end, it.kv_start, it.kv_len, it.worker, it.slot]
                      for it in p.items], dtype=np.int32).reshape(-1, 8)
    qptr = np.concatenate([[0], np.cumsum([len(q) for q in p.queues])]).astype(np.int32)
    qitems = np.array([m for q in p.queues for m in q], dtype=np.int32)
    mptr = np.concatenate([[0], np.cumsum([len(s) for s in p.merge_slots])]).astype(np.int32)
    mslots = np.array([s for ss in p.merge_slots for s in ss], dtype=np.int32)
    return {
        "tile_q": p.tile_q, "total_work": p.total_work, "chunk_limit": p.chunk_limit,
        "num_slots": p.num_slots, "group_size": p.group_size, "tiles": tiles, "items": items,
        "queue_ptr": qptr, "queue_items": qitems, "worker_cost": np.array(p.worker_cost, dtype=np.int64),
        "merge_tiles": np.array(p.merge_tiles, dtype=np.int32), "merge_ptr": mptr, "merge_slots": mslots,
        "tile_lo": np.array([t.lo for t in p.tiles], dtype=np.int32),
    }


def _assert_same(lib_plan, oracle_plan):
    a = lib_plan.export()
    b = _oracle_as_export(oracle_plan)
    for k, v in b.items():
        if isinstance(v, np.ndarray):
            assert np.array_equal(a[k].reshape(v.shape), v), k
        else:
            assert a[k] == v, k


def _lib_plan(kv_lens, qo_lens, Hq, Hk, C_, P=16, tq=0, causal=False, alpha=2, beta=1, d=128, window_left=-1):
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    ip, ix, last = I.page_table_from_lengths(kv_lens, P, np.arange(int(((kv_lens + P - 1) // P).sum())))
    qo = None if qo_lens is None else np.concatenate([[0], np.cumsum(qo_lens)])
    return api.Plan(ip, ix, last, num_pages=max(len(ix), 1), num_qo_heads=Hq, num_kv_heads=Hk,
                    head_dim=d, page_size=P, qo_indptr=qo, causal=causal, num_workers=C_,
                    tile_q=tq, alpha=alpha, beta=beta, window_left=window_left)


@pytest.mark.parametrize("alpha,beta", [(0, 1), (2, 1)])
def test_lpt_example_bit_exact(alpha, beta):
    g = load_golden("lpt_example.json")
    lp = _lib_plan(g["kv_lens"], None, 1, 1, g["num_ctas"], P=1, alpha=alpha, beta=beta)
    op = PL.make_plan(g["kv_lens"], None, 1, 1, g["num_ctas"], alpha=alpha, beta=beta)
    _assert_same(lp, op)
    assert lp.export()["chunk_limit"] == g["expected_chunk_limit"]


@pytest.mark.parametrize("seed", range(60))
def test_random_plans_bit_exact(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(0, 14))
    kv = rng.integers(0, 5000, size=B)
    kv[rng.random(B) < 0.15] = 0
    qo = None if rng.random() < 0.4 else rng.integers(1, 400, size=B)
    Hk = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    C_ = int(rng.integers(1, 300))
    tq = int(rng.choice([0, 0, 16, 32, 128]))
    causal = bool(rng.random() < 0.5) and qo is not None
    alpha, beta = [(2, 1), (0, 1), (3, 2)][int(rng.integers(0, 3))]
    P = int(rng.choice([1, 4, 16]))
    lp = _lib_plan(kv, qo, Hk * g, Hk, C_, P=P, tq=tq, causal=causal, alpha=alpha, beta=beta)
    op = PL.make_plan(kv, qo, Hk * g, Hk, C_, tile_q=tq, causal=causal, alpha=alpha, beta=beta)
    _assert_same(lp, op)


@pytest.mark.parametrize("seed", range(40))
def test_random_window_plans_bit_exact(seed):
    """Sliding-window plans ("FlashInfer 原理" §⑧): tiles start at their first row's window,
    the total work sums the windowed ranges, chunks start at each tile's first visible key."""
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 12))
    kv = rng.integers(0, 3000, size=B)
    qo = None if rng.random() < 0.3 else rng.integers(1, 300, size=B)
    if qo is not None:
        kv = np.maximum(kv, qo)  # queries are the last positions of their request
    Hk = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 4, 8]))
    C_ = int(rng.integers(1, 300))
    tq = int(rng.choice([0, 16, 64, 128]))
    causal = bool(rng.random() < 0.7) and qo is not None
    w = int(rng.choice([0, 1, 31, 127, 1000, 5000]))
    P = int(rng.choice([1, 16]))
    lp = _lib_plan(kv, qo, Hk * g, Hk, C_, P=P, tq=tq, causal=causal, window_left=w)
    op = PL.make_plan(kv, qo, Hk * g, Hk, C_, tile_q=tq, causal=causal, window_left=w)
    _assert_same(lp, op)
    e = lp.export()
    assert e["window_left"] == w and e["logits_soft_cap"] == 0.0
    assert e["total_work"] == int((e["tiles"][:, 3] - e["tile_lo"]).sum())


def test_soft_cap_leaves_the_plan_unchanged():
    lens = I.decode_lengths(2)[:40]
    a = _lib_plan(lens, None, 32, 8, 64).export()
    b = api.Plan(*I.page_table_from_lengths(np.asarray(lens), 16, np.arange(int(((np.asarray(lens) + 15) // 16).sum()))),
                 num_pages=int(((np.asarray(lens) + 15) // 16).sum()), num_qo_heads=32, num_kv_heads=8,
                 head_dim=128, page_size=16, num_workers=64, logits_soft_cap=30.0).export()
    assert b["logits_soft_cap"] == 30.0
    for k in ("tiles", "items", "queue_items", "merge_slots", "tile_lo"):
        assert np.array_equal(a[k], b[k]), k


def test_workload_plans_bit_exact():
    lens = I.decode_lengths(0)
    lp = _lib_plan(lens, None, 32, 8, 256)
    op = PL.make_plan(lens, None, 32, 8, 256)
    _assert_same(lp, op)
    pl = np.random.default_rng(0).integers(256, 4096, size=16, endpoint=True)
    lp = _lib_plan(pl, pl, 32, 8, 64, causal=True)
    op = PL.make_plan(pl, pl, 32, 8, 64, causal=True)
    _assert_same(lp, op)


def test_workspace_bound_eq13():
    lens = I.decode_lengths(1)
    for C_ in (16, 100, 256, 1000):
        p = _lib_plan(lens, None, 32, 8, C_)
        e = p.export()
        assert e["num_slots"] < 2 * C_
        part = e["num_slots"] * e["tile_q"] * 8 * (128 + 1)
        assert part <= PL.partial_capacity_bound(C_, e["tile_q"], 8, 128)
        assert p.workspace_bytes() >= part * 4


def _desc_errors():
    good = dict(kv_indptr=[0, 2, 3], kv_indices=[0, 1, 2], last_page_len=[4, 1], num_pages=3,
                num_qo_heads=4, num_kv_heads=2, head_dim=128, page_size=4)
    cases = [
        dict(kv_indptr=[1, 2, 3]),
        dict(kv_indptr=[0, 3, 2]),
        dict(kv_indices=[0, 1, 3]),
        dict(kv_indices=[0, -1, 2]),
        dict(last_page_len=[5, 1]),
        dict(last_page_len=[0, 1]),
        dict(num_qo_heads=3),
        dict(page_size=0),
        dict(head_dim=0),
        dict(tile_q=24),
        dict(qo_indptr=[0, 2, 1]),
        dict(qo_indptr=[1, 2, 3]),
        dict(window_left=-2),  # window_size -1
        dict(logits_soft_cap=-1.0),
        dict(logits_soft_cap=float("nan")),
        dict(logits_soft_cap=float("inf")),
    ]
    return good, cases


@pytest.mark.parametrize("i", range(16))
def test_invalid_descriptions(i):
    good, cases = _desc_errors()
    kw = dict(good)
    kw.update(cases[i])
    ip, ix, last = kw.pop("kv_indptr"), kw.pop("kv_indices"), kw.pop("last_page_len")
    with pytest.raises(_lib.BsrError) as ei:
        api.Plan(ip, ix, last, **kw)
    assert ei.value.status == _lib.BSR_INVALID_ARG
    assert _lib.lib().bsr_last_error().decode()


def test_empty_request_must_have_zero_last():
    with pytest.raises(_lib.BsrError):
        api.Plan([0, 0], [], [1], num_pages=1, num_qo_heads=1, num_kv_heads=1, head_dim=128, page_size=4)
    p = api.Plan([0, 0], [], [0], num_pages=1, num_qo_heads=1, num_kv_heads=1, head_dim=128, page_size=4)
    e = p.export()
    assert e["items"].shape[0] == 0 and e["merge_tiles"].tolist() == [0]


def test_null_arguments_rejected_without_gpu():
    L = _lib.lib()
    assert L.bsr_plan_create(None, C.byref(C.c_void_p())) == _lib.BSR_INVALID_ARG
    n = C.c_size_t()
    assert L.bsr_plan_workspace_bytes(None, C.byref(n)) == _lib.BSR_INVALID_ARG
    p = _lib_plan([10], None, 4, 1, 4)
    # run calls before any upload are rejected on the host, before touching the GPU
    rc = L.bsr_run_decode(p.handle, C.c_void_p(1234), None, None, None, None, None, 1, 0.1, None)
    assert rc == _lib.BSR_INVALID_ARG
    assert "uploaded" in L.bsr_last_error().decode()
    assert L.bsr_debug_gather_rows(p.handle, None, None, None) == _lib.BSR_INVALID_ARG
    assert L.bsr_merge_state(None, None, None, None, None, None, -1, 1, 1, 1, None) == _lib.BSR_INVALID_ARG
    assert L.bsr_merge_state(None, None, None, None, None, None, 1, 1, 1, 7, None) == _lib.BSR_INVALID_ARG


def test_custom_mask_bits_in_the_plan_view():
    kv, qo = [40, 0, 17, 300], [3, 5, 17, 1]
    lp = _lib_plan(kv, qo, 8, 2, 16, P=4)
    assert lp.export()["custom_mask_bits"] == sum(a * b for a, b in zip(kv, qo))
    dp = _lib_plan([40, 0, 17], None, 8, 2, 16, P=4)
    assert dp.export()["custom_mask_bits"] == 57  # one query per request


def test_pack_custom_mask_layout():
    m0 = np.array([[1, 0, 1], [0, 1, 1]], dtype=bool)
    m1 = np.array([[1, 1]], dtype=bool)
    assert api.pack_custom_mask([m0, m1]).tolist() == [0b11110101]


def _raw_plan(desc):
    h = C.c_void_p()
    rc = _lib.lib().bsr_plan_create(C.byref(desc), C.byref(h))
    assert rc == _lib.BSR_OK, _lib.lib().bsr_last_error().decode()
    return h


def _view(h):
    v = _lib.PlanView()
    assert _lib.lib().bsr_plan_export(h, C.byref(v)) == _lib.BSR_OK
    items = np.ctypeslib.as_array(v.items, shape=(v.num_items * 8,)).copy() if v.num_items else np.zeros(0)
    lo = np.ctypeslib.as_array(v.tile_lo, shape=(v.num_tiles,)).copy() if v.num_tiles else np.zeros(0)
    return v.window_left, v.total_work, v.chunk_limit, items, lo


def test_zero_filled_description_means_no_window():
    """A C caller that zero-fills bsr_plan_desc and sets only the BSR arrays and sizes gets the
    unwindowed attention: window_size 0 is "no window" (a window of one key is window_size 1)."""
    kv = np.array([37, 0, 300, 5], dtype=np.int64)
    ip, ix, last = I.page_table_from_lengths(kv, 8, np.arange(int(((kv + 7) // 8).sum())))
    ip, ix, last = (np.ascontiguousarray(a, dtype=np.int32) for a in (ip, ix, last))
    qo = np.ascontiguousarray([0, 3, 3, 40, 41], dtype=np.int32)

    def desc(**kw):
        d = _lib.PlanDesc()  # ctypes zero-fills every field
        d.batch, d.num_pages, d.num_qo_heads, d.num_kv_heads = 4, len(ix), 8, 2
        d.head_dim, d.page_size, d.causal, d.num_workers = 128, 8, 1, 7
        d.kv_indptr, d.kv_indices = ip.ctypes.data_as(_lib.i32p), ix.ctypes.data_as(_lib.i32p)
        d.last_page_len, d.qo_indptr = last.ctypes.data_as(_lib.i32p), qo.ctypes.data_as(_lib.i32p)
        for k, v in kw.items():
            setattr(d, k, v)
        return d

    zero = _raw_plan(desc())
    try:
        wl, W, L, items, lo = _view(zero)
        assert wl == -1 and not lo.any()
        ref = api.Plan(ip, ix, last, num_pages=len(ix), num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=8,
                       qo_indptr=qo, causal=True, num_workers=7, window_left=-1)
        e = ref.export()
        assert (W, L) == (e["total_work"], e["chunk_limit"]) and np.array_equal(items, e["items"].reshape(-1))
        # and window_size 1 is the diagonal-only window of the pages' window_left = 0
        one = _raw_plan(desc(window_size=1))
        try:
            wl1, W1, L1, items1, lo1 = _view(one)
            e0 = api.Plan(ip, ix, last, num_pages=len(ix), num_qo_heads=8, num_kv_heads=2, head_dim=128,
                          page_size=8, qo_indptr=qo, causal=True, num_workers=7, window_left=0).export()
            assert wl1 == 0 and W1 == e0["total_work"] and np.array_equal(items1, e0["items"].reshape(-1))
            assert np.array_equal(lo1, e0["tile_lo"]) and lo1.any()
        finally:
            _lib.lib().bsr_plan_destroy(one)
    finally:
        _lib.lib().bsr_plan_destroy(zero)


def _cpu_tensors(p, pages=None, page_size=None, lse_shape=None, dtype="bfloat16"):
    import torch

    dt = getattr(torch, dtype)
    pages = p.num_pages if pages is None else pages
    P = p.page_size if page_size is None else page_size
    q = torch.zeros(p.total_q, p.num_qo_heads, p.head_dim, dtype=dt)
    k = torch.zeros(pages, P, p.num_kv_heads, p.head_dim, dtype=dt)
    lse = torch.zeros(*(lse_shape or (p.total_q, p.num_qo_heads)), dtype=torch.float32)
    return q, k, k.clone(), torch.zeros_like(q), lse


@pytest.mark.parametrize("bad", ["short_cache", "page_size", "lse_shape", "lse_dtype", "cpu"])
def test_binding_rejects_mismatched_buffers_before_launch(bad):
    """The binding checks every buffer against the plan before the C call: a cache with fewer
    pages than the plan indexes, a different page size, or a short LSE would otherwise reach the
    kernels as out-of-bounds reads or writes."""
    import torch

    p = _lib_plan([40, 3, 17], None, 8, 2, 4, P=4)
    kw = {"short_cache": dict(pages=p.num_pages - 1), "page_size": dict(page_size=8),
          "lse_shape": dict(lse_shape=(p.total_q - 1, p.num_qo_heads)), "lse_dtype": {}, "cpu": {}}[bad]
    q, k, v, o, lse = _cpu_tensors(p, **kw)
    if bad == "lse_dtype":
        lse = lse.to(torch.float64)
    ws = torch.zeros(16, dtype=torch.uint8)
    err = TypeError if bad == "lse_dtype" else ValueError
    with pytest.raises(err) as ei:
        api.run_decode(p, ws, q, k, v, o=o, lse=lse)
    if bad == "cpu":
        assert "device tensor" in str(ei.value)
    with pytest.raises(err):
        api.run_decode_e4m3(p, ws, q, k.to(torch.uint8) if bad != "lse_dtype" else k.to(torch.uint8),
                            v.to(torch.uint8), 1.0, 1.0, o=o, lse=lse)


def test_merge_state_binding_checks_every_lse():
    import torch

    o = torch.zeros(5, 4, 64)
    l = torch.zeros(5, 4)
    with pytest.raises(ValueError):
        api.merge_state(o, l, o, torch.zeros(4, 4))
    with pytest.raises(ValueError):
        api.merge_state(o, l, o, l, o_out=torch.zeros_like(o), lse_out=torch.zeros(5, 3))
    with pytest.raises(TypeError):
        api.merge_state(o, l, o, l.double())
    with pytest.raises(ValueError):  # right shapes, but host tensors
        api.merge_state(o, l, o, l)


def test_prefill_lpt_hand_worked_example_in_the_library():
    """The C++ planner against the hand-worked prefill schedule itself (not only against the
    oracle's copy of the rule)."""
    g = load_golden("lpt_prefill_hand.json")
    lp = _lib_plan(g["kv_lens"], g["qo_lens"], g["num_qo_heads"], g["num_kv_heads"], g["num_workers"], P=2,
                   tq=g["tile_q"], causal=g["causal"], alpha=g["alpha"], beta=g["beta"])
    e = lp.export()
    assert e["tiles"][:, :4].tolist() == g["expected_tiles"]
    assert (e["total_work"], e["chunk_limit"]) == (g["expected_total_work"], g["expected_chunk_limit"])
    assert e["items"][:, [1, 4, 5]].tolist() == g["expected_items"]
    qp, qi = e["queue_ptr"], e["queue_items"]
    assert [qi[qp[w]:qp[w + 1]].tolist() for w in range(g["num_workers"])] == g["expected_queues"]
    assert e["worker_cost"].tolist() == g["expected_worker_cost"]
    assert e["items"][:, 7].tolist() == g["expected_slots"]
    assert e["merge_tiles"].tolist() == g["expected_merge_tiles"]
    mp = e["merge_ptr"]
    assert [e["merge_slots"][mp[k]:mp[k + 1]].tolist() for k in range(len(mp) - 1)] == g["expected_merge_slots"]


def _composable_lib_and_oracle(levels, Hq, Hk, C_, P=16, seed=0):
    """levels: list of (kv_lens, qo_lens or None).  Pages: one permutation of the pool shared by
    the levels (only the lengths matter to the plan)."""
    rng = np.random.default_rng(seed)
    need = sum(int(((np.asarray(kv) + P - 1) // P).sum()) for kv, _ in levels)
    pool = max(need, 1)
    perm = rng.permutation(pool)
    descs, off = [], 0
    for kv, qo in levels:
        kv = np.asarray(kv, dtype=np.int64)
        n = int(((kv + P - 1) // P).sum())
        ip, ix, la = I.page_table_from_lengths(kv, P, perm[off:off + n])
        off += n
        d = dict(kv_indptr=ip, kv_indices=ix, last_page_len=la)
        if qo is not None:
            d["qo_indptr"] = np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)
        descs.append(d)
    lp = api.ComposablePlan(descs, num_pages=pool, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=128, page_size=P,
                            num_workers=C_)
    op = PL.make_composable_plan(levels, Hq, Hk, C_)
    return lp, op


def _assert_composable_same(lp, op):
    e = lp.export()
    assert e["num_levels"] == len(op.level_req_start) - 1
    assert e["level_req_start"].tolist() == op.level_req_start
    assert (e["tile_q"], e["total_work"], e["chunk_limit"], e["num_slots"]) == \
           (op.tile_q, op.total_work, op.chunk_limit, op.num_slots)
    assert e["tiles"][:, :4].tolist() == [[t.req, t.row_start, t.row_end, t.vis] for t in op.tiles]
    assert e["items"].tolist() == [[it.req, it.tile, it.row_start, it.row_end, it.kv_start, it.kv_len, it.worker,
                                    it.slot] for it in op.items]
    qp, qi = e["queue_ptr"], e["queue_items"]
    assert [qi[qp[w]:qp[w + 1]].tolist() for w in range(op.num_workers)] == op.queues
    assert e["worker_cost"].tolist() == op.worker_cost
    mp = e["merge_ptr"]
    assert e["merge_tiles"].tolist() == list(range(len(op.units)))
    got = [list(zip(e["merge_slots"][mp[k]:mp[k + 1]].tolist(), e["merge_row_off"][mp[k]:mp[k + 1]].tolist()))
           for k in range(len(mp) - 1)]
    assert got == [list(u) for u in op.units]


@pytest.mark.parametrize("seed", range(30))
def test_random_composable_plans_bit_exact(seed):
    rng = np.random.default_rng(100 + seed)
    g = int(rng.choice([1, 2, 4, 8, 16]))
    Hk = int(rng.choice([1, 2, 8]))
    nq = int(rng.integers(1, 40))
    levels = []
    for _ in range(int(rng.integers(1, 4))):
        # a random grouping of the nq queries into block rows (some possibly empty)
        cuts = np.sort(rng.integers(0, nq + 1, size=int(rng.integers(0, 6))))
        qo = np.diff(np.concatenate([[0], cuts, [nq]]))
        kv = rng.integers(0, 3000, size=len(qo))
        kv[rng.random(len(qo)) < 0.15] = 0
        levels.append((kv, None if (rng.random() < 0.3 and np.all(qo == 1)) else qo))
    if rng.random() < 0.5:
        levels.append((rng.integers(0, 900, size=nq), None))  # private rows, one query each
    C_ = int(rng.integers(1, 300))
    lp, op = _composable_lib_and_oracle(levels, Hk * g, Hk, C_, P=int(rng.choice([1, 4, 16])), seed=seed)
    _assert_composable_same(lp, op)


def test_composable_shared_prefix_plan_bit_exact():
    """The composable shared-prefix workload: 16 groups of 4 sharing a 2048-token prefix, private
    suffixes U[128, 1024], at 256 workers."""
    b = I.shared_prefix_decode(seed=0, poison=False)
    levels = [(np.full(b.groups, b.prefix_len), np.full(b.groups, b.per_group)), (b.suffix_lens, None)]
    lp, op = _composable_lib_and_oracle(levels, 32, 8, 256)
    _assert_composable_same(lp, op)


def test_composable_rejects_mismatched_levels():
    base = dict(kv_indptr=[0, 1], kv_indices=[0], last_page_len=[3])
    bad = [
        [base, dict(kv_indptr=[0, 1, 2], kv_indices=[0, 1], last_page_len=[1, 1])],  # 1 query vs 2
        [dict(base, qo_indptr=[0, 2]), dict(kv_indptr=[0, 1, 1], kv_indices=[1], last_page_len=[2, 0])],  # g = 3
    ]
    with pytest.raises(_lib.BsrError):
        api.ComposablePlan(bad[0], num_pages=4, num_qo_heads=4, num_kv_heads=1, head_dim=128, page_size=4)
    with pytest.raises(_lib.BsrError):
        api.ComposablePlan(bad[1], num_pages=4, num_qo_heads=3, num_kv_heads=1, head_dim=128, page_size=4)


def test_null_kv_indices_plans_a_contiguous_cache():
    """kv_indices NULL describes a contiguous cache (request i's pages are kv_indptr[i] ..
    kv_indptr[i+1] - 1): planned exactly as with the identity page table written out, and a
    pool with fewer pages than kv_indptr[B] is rejected on the host."""
    for P, qo in ((16, None), (1, None), (12, [3, 1, 40, 2, 7])):
        kv = np.array([37, 0, 300, 5, 1000], dtype=np.int64)
        n = int(((kv + P - 1) // P).sum())
        ip, ix, last = I.page_table_from_lengths(kv, P, np.arange(n))
        assert np.array_equal(ix, np.arange(n))
        qo_ip = None if qo is None else np.concatenate([[0], np.cumsum(qo)])
        kw = dict(num_pages=n + 5, num_qo_heads=8, num_kv_heads=2, head_dim=128, page_size=P, qo_indptr=qo_ip,
                  causal=qo is not None, num_workers=9)
        a, b = api.Plan(ip, ix, last, **kw), api.Plan(ip, None, last, **kw)
        ea, eb = a.export(), b.export()
        assert ea.keys() == eb.keys()
        for k in ea:
            assert np.array_equal(np.asarray(ea[k]), np.asarray(eb[k])), k
        assert a.workspace_bytes() == b.workspace_bytes()
        kw["num_pages"] = n - 1
        with pytest.raises(_lib.BsrError, match="outside"):
            api.Plan(ip, None, last, **kw)
