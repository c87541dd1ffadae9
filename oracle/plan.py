"""Load-balanced split-KV work partition, written out step by step.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The partition is the longest-processing-time greedy of FlashInfer's runtime
scheduler as the pages describe it:

* "FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for LLM
  Inference Serving", §VIII.2 (chunk limit from total work over the CTA count, chunk
  every query tile's KV, sort descending, min-heap of CTAs keyed by accumulated cost,
  cost alpha * l_q + beta * l_kv), §VIII.3 (fixed aggregation order, no atomics),
  §VIII.5 (partial -> final reduction map, Figure 6) and §VI.2 (query tile: smallest
  size at least the average packed query length).
* "FlashInfer 原理", §⑦ (packed query length = qo_len x group size) and §⑨ (worked
  example with KV lengths [1000, 100, 100, 50] on 4 CTAs, ceil for the chunk limit;
  short requests write final outputs directly).
* "FlashInfer: Making Attention Fit the Serving Workload", §6.1 (eq. 10 total work,
  eq. 11 linear cost) and §6.2 (integer chunk limit max(1, ceil(W / C)), ties broken
  by a stable id, heap of (cost, CTA id), ordered partial list per output tile).

Readings taken where the pages leave a detail open:
the query-tile set is {16, 32, 64, 128} (a tile is a multiple of the 16-row matrix
instruction; 128 when the average exceeds 64); the per-item cost charges the query
positions of the item's own tile (one for a decode request, at most T_q / g for a
prefill tile) plus its chunk length; chunks are counted in tokens and may start inside a page; a causal
tile's visible KV range ends at the tile's last query position, and with a sliding window of
w keys it starts at the window's start for the tile's first query position (the total work
then sums the tiles' windowed ranges instead of eq. 10's full lengths); ties in the heap go
to the lower worker id; a tile with exactly one chunk writes its final output, the
chunks of split tiles get partial slots 0, 1, 2, ... in assignment order, and each
split tile's reduction list orders its slots by KV start.
"""
from __future__ import annotations

import heapq
from dataclasses import dataclass, field
from typing import List

TILE_SET = (16, 32, 64, 128)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class Tile:
    req: int
    row_start: int  # packed rows [row_start, row_end) of the request
    row_end: int
    vis: int  # end of the tile's visible KV range
    lo: int = 0  # start of the tile's visible KV range (> 0 only with a sliding window)
    items: List[int] = field(default_factory=list)  # creation-order item ids


@dataclass
class Item:
    req: int
    tile: int
    row_start: int
    row_end: int
    kv_start: int
    kv_len: int
    worker: int = -1
    slot: int = -1


@dataclass
class Plan:
    group_size: int
    tile_q: int
    total_work: int
    chunk_limit: int
    num_workers: int
    tiles: List[Tile]
    items: List[Item]
    queues: List[List[int]]
    worker_cost: List[int]
    merge_tiles: List[int]  # tiles that the merge pass writes (split or empty)
    merge_slots: List[List[int]]  # ordered slot list per merge tile
    num_slots: int


def tile_positions(item, g):
    """Query positions covered by the packed rows [row_start, row_end) of a tile."""
    return (item.row_end - 1) // g - item.row_start // g + 1


def choose_tile_q(packed_lens, tile_q=0):
    """Query tile: smallest tile >= the average packed query length (rounded up)."""
    if tile_q:
        return int(tile_q)
    B = len(packed_lens)
    avg = ceil_div(sum(packed_lens), B) if B else 0
    for t in TILE_SET:
        if t >= avg:
            return t
    return TILE_SET[-1]


def make_plan(
    kv_lens,
    qo_lens,
    num_qo_heads,
    num_kv_heads,
    num_workers,
    tile_q=0,
    alpha=2,
    beta=1,
    causal=False,
    window_left=-1,
):
    """Build the partition for requests with the given query and KV lengths.

    ``window_left`` >= 0: sliding window; the visible range of a tile starts at
    max(0, l_kv - l_qo + first_pos - window_left) (its first row's window start)."""
    kv_lens = [int(x) for x in kv_lens]
    B = len(kv_lens)
    qo_lens = [1] * B if qo_lens is None else [int(x) for x in qo_lens]
    assert num_qo_heads % num_kv_heads == 0 and num_workers >= 1
    g = num_qo_heads // num_kv_heads

    # packed (GQA-fused) query length of every request
    pq = [lq * g for lq in qo_lens]
    T = choose_tile_q(pq, tile_q)

    # query tiles of every request and their visible KV range
    tiles: List[Tile] = []
    for i in range(B):
        for j in range(ceil_div(pq[i], T)):
            r0 = j * T
            r1 = min(r0 + T, pq[i])
            last_pos = (r1 - 1) // g
            if causal:
                vis = max(0, min(kv_lens[i], kv_lens[i] - qo_lens[i] + last_pos + 1))
            else:
                vis = kv_lens[i]
            lo = 0
            if window_left >= 0:
                lo = min(vis, max(0, kv_lens[i] - qo_lens[i] + r0 // g - window_left))
            tiles.append(Tile(i, r0, r1, vis, lo))

    # total work (eq. 10; with a window, the tiles' windowed ranges) and the chunk limit
    if window_left >= 0:
        W = sum(t.vis - t.lo for t in tiles)
    else:
        W = sum(ceil_div(pq[i], T) * kv_lens[i] for i in range(B))
    L = max(1, ceil_div(W, num_workers)) if (B > 0 and W > 0) else 0

    # work items: chunks of each tile's visible range, in creation order
    items: List[Item] = []
    if L > 0:
        for t_id, t in enumerate(tiles):
            s = t.lo
            while s < t.vis:
                n = min(L, t.vis - s)
                t.items.append(len(items))
                items.append(Item(t.req, t_id, t.row_start, t.row_end, s, n))
                s += L

    # longest first; Python's sort is stable, so equal lengths keep creation order
    order = sorted(range(len(items)), key=lambda m: -items[m].kv_len)

    # least-loaded worker first, ties to the lower worker id
    heap = [(0, w) for w in range(num_workers)]
    heapq.heapify(heap)
    queues: List[List[int]] = [[] for _ in range(num_workers)]
    cost = [0] * num_workers
    for m in order:
        c, w = heapq.heappop(heap)
        queues[w].append(m)
        items[m].worker = w
        c += alpha * tile_positions(items[m], g) + beta * items[m].kv_len
        cost[w] = c
        heapq.heappush(heap, (c, w))

    # partial slots for chunks of split tiles, numbered in assignment order
    slot = 0
    for m in order:
        if len(tiles[items[m].tile].items) > 1:
            items[m].slot = slot
            slot += 1

    # reduction map: split tiles fold their slots by ascending KV start; empty tiles
    # (nothing visible) are written as empty states by the same pass
    merge_tiles, merge_slots = [], []
    for t_id, t in enumerate(tiles):
        if len(t.items) == 1:
            continue
        merge_tiles.append(t_id)
        ids = sorted(t.items, key=lambda m: items[m].kv_start)
        merge_slots.append([items[m].slot for m in ids])

    return Plan(
        group_size=g,
        tile_q=T,
        total_work=W,
        chunk_limit=L,
        num_workers=num_workers,
        tiles=tiles,
        items=items,
        queues=queues,
        worker_cost=cost,
        merge_tiles=merge_tiles,
        merge_slots=merge_slots,
        num_slots=slot,
    )


def partial_capacity_bound(num_workers, tile_q, num_heads, head_dim):
    """Eq. 13 of the review (§6.5): E_partial <= 2 C T_q H (d + 1) scalars.

    With query tiles counted in query positions, H is the number of query heads (the
    equation as printed).  With GQA-packed tiles (T_q packed rows of one KV head), the
    same count reads 2 C T_q H_kv (d + 1): pass the KV head count.
    """
    return 2 * num_workers * tile_q * num_heads * (head_dim + 1)


@dataclass
class ComposablePlan:
    group_size: int
    tile_q: int
    total_work: int
    chunk_limit: int
    num_workers: int
    level_req_start: List[int]  # first flattened request of each level (+ the total)
    tiles: List[Tile]  # every level's tiles; Tile.req is the flattened request index
    items: List[Item]
    queues: List[List[int]]
    worker_cost: List[int]
    units: List[List[tuple]]  # per query: (slot, row offset inside the slot's tile), in fold order
    num_slots: int


def make_composable_plan(levels, num_qo_heads, num_kv_heads, num_workers, alpha=2, beta=1, tile_q=16):
    """Partition of a composable format: several BSR views ("levels") of one KV pool over the
    same queries, whose attention states are merged per query ("FlashInfer: Engineering a
    Customizable, Block-Sparse Attention Engine for LLM Inference Serving" §IV.6; "FlashInfer
    原理" §⑤; eq. 6 of "FlashInfer: Making Attention Fit the Serving Workload").

    ``levels``: list of (kv_lens, qo_lens) per level, qo_lens None for one query per request;
    every level holds the same queries, numbered in request order.  The pages leave the joint
    schedule open; the reading taken here: each level's block rows are tiled exactly as
    ``make_plan`` tiles a non-causal batch (tile_q packed rows), the tiles of all levels form one
    batch (levels in order) for the partition steps of ``make_plan`` -- total work (the levels'
    eq. 10 sums), one chunk limit, creation-order chunks, one stable descending sort, one heap --
    and every chunk writes a partial state (slots in assignment order).  Query q's reduction list
    walks the levels in order and, in each, the chunks of the tile holding q's rows in KV order;
    a chunk's row offset is the tile row of q's first packed row.
    """
    g = num_qo_heads // num_kv_heads
    assert tile_q % g == 0, "a query's packed rows must not straddle two tiles"
    per_level = [make_plan(kv, qo, num_qo_heads, num_kv_heads, 1, tile_q=tile_q, alpha=alpha, beta=beta)
                 for kv, qo in levels]
    level_req_start = [0]
    tiles: List[Tile] = []
    W = 0
    for lp, (kv, qo) in zip(per_level, levels):
        base = level_req_start[-1]
        for t in lp.tiles:
            tiles.append(Tile(base + t.req, t.row_start, t.row_end, t.vis))
        level_req_start.append(base + len(kv))
        W += lp.total_work
    L = max(1, ceil_div(W, num_workers)) if W > 0 else 0

    items: List[Item] = []
    if L > 0:
        for t_id, t in enumerate(tiles):
            s = 0
            while s < t.vis:
                t.items.append(len(items))
                items.append(Item(t.req, t_id, t.row_start, t.row_end, s, min(L, t.vis - s)))
                s += L
    order = sorted(range(len(items)), key=lambda m: -items[m].kv_len)
    heap = [(0, w) for w in range(num_workers)]
    heapq.heapify(heap)
    queues: List[List[int]] = [[] for _ in range(num_workers)]
    cost = [0] * num_workers
    for m in order:
        c, w = heapq.heappop(heap)
        queues[w].append(m)
        items[m].worker = w
        c += alpha * tile_positions(items[m], g) + beta * items[m].kv_len
        cost[w] = c
        heapq.heappush(heap, (c, w))
    for slot, m in enumerate(order):
        items[m].slot = slot

    # per query: in every level, the tile that holds its rows
    qo0 = levels[0][1]
    total_q = len(levels[0][0]) if qo0 is None else int(sum(qo0))
    units = [[] for _ in range(total_q)]
    t_id = 0
    for li, (kv, qo) in enumerate(levels):
        qo = [1] * len(kv) if qo is None else [int(x) for x in qo]
        q0 = 0
        for i in range(len(kv)):
            nt = ceil_div(qo[i] * g, tile_q)
            for pos in range(qo[i]):
                row = pos * g
                t = tiles[t_id + row // tile_q]
                for m in sorted(t.items, key=lambda m: items[m].kv_start):
                    units[q0 + pos].append((items[m].slot, row - t.row_start))
            t_id += nt
            q0 += qo[i]
        assert q0 == total_q, "every level must hold the same queries"
    return ComposablePlan(g, tile_q, W, L, num_workers, level_req_start, tiles, items, queues, cost, units,
                          len(order))
