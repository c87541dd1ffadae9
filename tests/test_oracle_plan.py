"""Pins of the oracle planner: the pages' worked examples plus invariants."""
import math

import numpy as np
import pytest

from oracle import plan as PL
from tests.conftest import load_golden


@pytest.mark.parametrize("alpha,beta", [(0, 1), (2, 1)])
def test_lpt_worked_example(alpha, beta):
    g = load_golden("lpt_example.json")
    p = PL.make_plan(g["kv_lens"], None, 1, 1, g["num_ctas"], alpha=alpha, beta=beta)
    assert p.total_work == g["total_work"]
    assert p.chunk_limit == g["expected_chunk_limit"]
    a_chunks = [it.kv_len for it in p.items if it.req == 0]
    assert a_chunks == g["expected_chunks_of_A"]
    order = sorted(range(len(p.items)), key=lambda m: -p.items[m].kv_len)
    assert [p.items[m].kv_len for m in order] == g["expected_sorted_lengths"]
    names = {}
    for m, it in enumerate(p.items):
        names[m] = "ABCD"[it.req] + (str(it.kv_start // p.chunk_limit) if it.req == 0 else "")
    got = [[names[m] for m in q] for q in p.queues]
    assert got == g["expected_cta_contents"]
    assert sum(p.items[m].kv_len for m in p.queues[3]) == g["expected_cta3_total"]
    if alpha == 0:
        assert p.worker_cost[3] == g["expected_cta3_total"]
    # A was split into four chunks and merges in KV order; B, C, D write directly
    assert len(p.merge_tiles) == 1 and p.tiles[p.merge_tiles[0]].req == 0
    slots = p.merge_slots[0]
    starts = [next(it.kv_start for it in p.items if it.slot == s) for s in slots]
    assert starts == sorted(starts) == [0, 313, 626, 939]
    assert all(it.slot == -1 for it in p.items if it.req != 0)


def test_tile_choice_example():
    g = load_golden("tile_choice.json")
    assert PL.choose_tile_q(g["qo_lens"]) == g["expected_tile"]
    assert PL.choose_tile_q([200]) == 128 and PL.choose_tile_q([17]) == 32


def test_gqa_packing_examples():
    g = load_golden("gqa_packing.json")
    e = g["eq3_example"]
    p = PL.make_plan([10], [e["L_q"]], e["g"], 1, 1, tile_q=16)
    assert p.tiles[0].row_end - p.tiles[0].row_start == e["expected_rows"]
    o = g["overview_example"]
    p = PL.make_plan([10], [o["qo_len"]], o["g"] * 2, 2, 1)
    assert p.tiles[0].row_end == o["expected_packed"] and p.tile_q == o["expected_tile"]


def test_capacity_arithmetic():
    g = load_golden("capacity.json")
    n = PL.partial_capacity_bound(g["C"], g["T_q"], g["H_q"], g["d"])
    assert n == g["expected_elements"]
    mib, tol = g["expected_mib_at_4_bytes"]
    assert abs(n * 4 / 2**20 - mib) <= tol


def _random_case(rng):
    B = int(rng.integers(0, 12))
    kv = rng.integers(0, 3000, size=B)
    if rng.random() < 0.3:
        kv[rng.random(B) < 0.3] = 0
    causal = bool(rng.random() < 0.5)
    qo = None if rng.random() < 0.4 else rng.integers(1, 300, size=B)
    Hk = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    C = int(rng.integers(1, 70))
    tq = int(rng.choice([0, 0, 16, 64]))
    return kv, qo, Hk * g, Hk, C, tq, causal


@pytest.mark.parametrize("seed", range(40))
def test_invariants(seed):
    rng = np.random.default_rng(seed)
    kv, qo, Hq, Hk, C, tq, causal = _random_case(rng)
    p = PL.make_plan(kv, qo, Hq, Hk, C, tile_q=tq, causal=causal)
    again = PL.make_plan(kv, qo, Hq, Hk, C, tile_q=tq, causal=causal)
    assert p == again  # identical input -> identical plan
    g = Hq // Hk
    qol = [1] * len(kv) if qo is None else list(qo)
    # every visible (tile, token) covered exactly once, chunks <= L
    for t_id, t in enumerate(p.tiles):
        cov = np.zeros(t.vis, dtype=int)
        for m in t.items:
            it = p.items[m]
            assert it.tile == t_id and 0 < it.kv_len <= p.chunk_limit
            cov[it.kv_start : it.kv_start + it.kv_len] += 1
        assert np.all(cov == 1)
        last_pos = (t.row_end - 1) // g
        l_kv, l_qo = int(kv[t.req]), int(qol[t.req])
        exp_vis = max(0, min(l_kv, l_kv - l_qo + last_pos + 1)) if causal else l_kv
        assert t.vis == exp_vis
    # every item assigned, each worker's queue holds it once
    seen = sorted(m for q in p.queues for m in q)
    assert seen == list(range(len(p.items)))
    # greedy property: each item went to a least-loaded worker at its turn
    order = sorted(range(len(p.items)), key=lambda m: -p.items[m].kv_len)
    load = [0] * C
    for m in order:
        w = p.items[m].worker
        assert load[w] == min(load) and w == load.index(min(load))
        it = p.items[m]
        positions = (it.row_end - 1) // g - it.row_start // g + 1
        assert 1 <= positions <= min(qol[it.req], p.tile_q)
        load[w] += 2 * positions + it.kv_len
    assert load == p.worker_cost
    # slots: exactly the chunks of split tiles, numbered 0.. in assignment order
    split = [m for m in order if len(p.tiles[p.items[m].tile].items) > 1]
    assert [p.items[m].slot for m in split] == list(range(len(split)))
    assert p.num_slots == len(split)
    # reduction map lists split and empty tiles in creation order, slots by kv_start
    exp_tiles = [i for i, t in enumerate(p.tiles) if len(t.items) != 1]
    assert p.merge_tiles == exp_tiles
    for t_id, slots in zip(p.merge_tiles, p.merge_slots):
        starts = [next(it.kv_start for it in p.items if it.slot == s) for s in slots]
        assert starts == sorted(starts) and len(slots) == len(p.tiles[t_id].items)
    # eq. 13 in packed rows: partial slots < 2 C, so partial scalars <= 2 C T_q H_kv (d+1)
    assert p.num_slots <= 2 * C
    d = 128
    assert p.num_slots * p.tile_q * Hk * (d + 1) <= PL.partial_capacity_bound(C, p.tile_q, Hk, d)


def test_empty_batch_and_zero_work():
    p = PL.make_plan([], None, 4, 1, 8)
    assert p.items == [] and p.tiles == [] and p.chunk_limit == 0
    p = PL.make_plan([0, 0], None, 4, 1, 8)
    assert p.items == [] and p.merge_tiles == [0, 1] and p.merge_slots == [[], []]


def test_causal_long_query_short_kv_has_empty_tiles():
    # bottom-right alignment: with 64 queries and 8 keys, the first 56 positions see nothing
    p = PL.make_plan([8], [64], 1, 1, 4, tile_q=16, causal=True)
    assert [t.vis for t in p.tiles] == [0, 0, 0, 8]
    assert p.merge_tiles[:3] == [0, 1, 2]


def _prefill_hand_plan(tp=None, monkeypatch=None):
    g = load_golden("lpt_prefill_hand.json")
    if tp is not None:
        monkeypatch.setattr(PL, "tile_positions", tp)
    return g, PL.make_plan(g["kv_lens"], g["qo_lens"], g["num_qo_heads"], g["num_kv_heads"], g["num_workers"],
                           tile_q=g["tile_q"], alpha=g["alpha"], beta=g["beta"], causal=g["causal"])


def _matches_prefill_golden(g, p):
    items = [[it.tile, it.kv_start, it.kv_len] for it in p.items]
    order = sorted(range(len(p.items)), key=lambda m: -p.items[m].kv_len)
    return (
        [[t.req, t.row_start, t.row_end, t.vis] for t in p.tiles] == g["expected_tiles"]
        and [PL.tile_positions(t, p.group_size) for t in p.tiles] == g["expected_tile_positions"]
        and p.total_work == g["expected_total_work"]
        and p.chunk_limit == g["expected_chunk_limit"]
        and items == g["expected_items"]
        and order == g["expected_sorted_items"]
        and p.queues == g["expected_queues"]
        and p.worker_cost == g["expected_worker_cost"]
        and [it.slot for it in p.items] == g["expected_slots"]
        and p.merge_tiles == g["expected_merge_tiles"]
        and p.merge_slots == g["expected_merge_slots"]
    )


def test_prefill_lpt_hand_worked_example():
    """The prefill item cost (query positions of the item's own tile) against a schedule worked
    out by hand (tests/golden/lpt_prefill_hand.json)."""
    g, p = _prefill_hand_plan()
    assert _matches_prefill_golden(g, p)
    costs = [2 * PL.tile_positions(it, p.group_size) + it.kv_len for it in p.items]
    assert costs == g["expected_item_costs"]


# plausible mistakes in the item cost, each planted in the oracle: the whole request's query
# length charged to every tile, the row count divided by g (floor or ceil), the position span
# without its + 1
_WRONG_POSITIONS = {
    "request_qo_len": None,  # filled in below (needs the plan's requests)
    "rows_floor_div_g": lambda it, g: (it.row_end - it.row_start) // g,
    "rows_ceil_div_g": lambda it, g: -(-(it.row_end - it.row_start) // g),
    "span_without_plus_one": lambda it, g: (it.row_end - 1) // g - it.row_start // g,
}


@pytest.mark.parametrize("variant", sorted(_WRONG_POSITIONS))
def test_prefill_lpt_golden_rejects_wrong_cost(variant, monkeypatch):
    gold = load_golden("lpt_prefill_hand.json")
    tp = _WRONG_POSITIONS[variant]
    if tp is None:
        qo = gold["qo_lens"]
        tp = lambda it, g: qo[it.req]  # noqa: E731
    g, p = _prefill_hand_plan(tp, monkeypatch)
    assert not _matches_prefill_golden(g, p), variant


def test_composable_plan_single_level_is_the_plain_schedule():
    """One level: the same tiles, chunks, queues and costs as make_plan (non-causal, 16-row tiles);
    only every chunk takes a slot, and each query's list is its tile's chunks in KV order."""
    kv, qo = [70, 0, 300, 33], [5, 2, 9, 1]
    cp = PL.make_composable_plan([(kv, qo)], 8, 2, 5)
    p = PL.make_plan(kv, qo, 8, 2, 5, tile_q=16)
    assert [(t.req, t.row_start, t.row_end, t.vis) for t in cp.tiles] == \
           [(t.req, t.row_start, t.row_end, t.vis) for t in p.tiles]
    assert [(it.tile, it.kv_start, it.kv_len, it.worker) for it in cp.items] == \
           [(it.tile, it.kv_start, it.kv_len, it.worker) for it in p.items]
    assert cp.queues == p.queues and cp.worker_cost == p.worker_cost
    assert sorted(it.slot for it in cp.items) == list(range(len(cp.items)))
    # g = 4; queries 0-4 are request 0, 5-6 request 1 (no keys), 7-15 request 2, 16 request 3.
    # Query 8 = request 2, position 1: rows 4..7 of request 2's first tile
    t = next(t for t in cp.tiles if t.req == 2 and t.row_start == 0)
    assert [r for _, r in cp.units[8]] == [4] * len(t.items)
    assert [s for s, _ in cp.units[8]] == [cp.items[m].slot for m in sorted(t.items, key=lambda m: cp.items[m].kv_start)]
    # query 11 = request 2, position 4: rows 16..19 = row 0 of request 2's second tile
    t2 = next(t for t in cp.tiles if t.req == 2 and t.row_start == 16)
    assert [r for _, r in cp.units[11]] == [0] * len(t2.items)
    assert cp.units[5] == [] and cp.units[6] == []  # request 1 has no keys


def test_composable_plan_by_hand():
    """Two levels over 4 queries (g = 2): level 0 is one block row of all 4 queries over 6 keys,
    level 1 one row per query over 2, 0, 5 and 1 keys; 3 workers."""
    cp = PL.make_composable_plan([([6], [4]), ([2, 0, 5, 1], None)], 4, 2, 3, alpha=2, beta=1)
    # tiles: level 0 one tile of 8 rows (vis 6); level 1 four tiles of 2 rows (vis 2, 0, 5, 1)
    assert [(t.req, t.row_start, t.row_end, t.vis) for t in cp.tiles] == \
           [(0, 0, 8, 6), (1, 0, 2, 2), (2, 0, 2, 0), (3, 0, 2, 5), (4, 0, 2, 1)]
    # W = 6 + (2 + 0 + 5 + 1) = 14, L = ceil(14 / 3) = 5
    assert (cp.total_work, cp.chunk_limit) == (14, 5)
    # chunks: m0 t0 [0,5), m1 t0 [5,6), m2 t1 [0,2), m3 t3 [0,5), m4 t4 [0,1)
    assert [(it.tile, it.kv_start, it.kv_len) for it in cp.items] == [(0, 0, 5), (0, 5, 1), (1, 0, 2), (3, 0, 5), (4, 0, 1)]
    # sorted: m0 (5), m3 (5), m2 (2), m1 (1), m4 (1); costs 2 * positions + length: m0 2*4+5 = 13,
    # m3 2*1+5 = 7, m2 2+2 = 4, m1 8+1 = 9, m4 2+1 = 3
    # heap: m0 -> w0 (13), m3 -> w1 (7), m2 -> w2 (4), m1 -> w2 (13), m4 -> w1 (10)
    assert cp.queues == [[0], [3, 4], [2, 1]] and cp.worker_cost == [13, 10, 13]
    assert [it.slot for it in cp.items] == [0, 3, 2, 1, 4]
    # query 0: level 0 rows 0..1 (slots of m0, m1 in KV order, offset 0), level 1 request 0 (m2)
    assert cp.units == [[(0, 0), (3, 0), (2, 0)], [(0, 2), (3, 2)], [(0, 4), (3, 4), (1, 0)], [(0, 6), (3, 6), (4, 0)]]
