"""Host model of the bf16 prefill kernels' page-window lookups and LDS-DMA wait accounting.

The prefill kernels (block_sparse_paged_bsr_amd/csrc/kernels/attn_prefill_bf16.hip) stage a
window of up to kPageWindow page ids of the request's page list in LDS, look token pages up
there, and gather K/V rows into LDS rings with asynchronous DMA loads whose completion they wait
for with hand-counted `vmcnt` limits.  A page id read from outside the filled window, or a wait
that lets a tile's loads still be in flight when a barrier publishes it, would turn into a wild
address or a stale tile on the GPU.  This module replays, on the CPU, the sequence of window
fills, page lookups (general and fast forms), DMA issues, waits, barriers and ring reads that
each kernel shape performs for the work items of a plan, and asserts:

* every window lookup index lies in [0, filled entries) for every token a lane loads (page_no
  is monotone in the token, so a tile's first and last token bound all of its lanes);
* the fast (page size divides 32) lookup indices and in-page row offsets equal the general ones;
* every DMA targets a tile that exists, into a ring slot whose previous tile was last read
  before the barrier that precedes the issue, with no other load in flight into that slot;
* at every barrier the tiles the following stream reads have completed (loads of one wave
  complete in issue order, so "at most n batches in flight" completes all but the n youngest);
* the batches per step and the wait limits agree with the kernel's compile-time constants
  (kDmaBatchesPerStep, kMaxBatchesInFlight).

The plans come from the library's own planner (bsr_plan_export), so the model runs the work
items the kernels run.
"""
import functools
import os
import re

import numpy as np
import pytest

from block_sparse_paged_bsr_amd import _lib
from block_sparse_paged_bsr_amd import api
import workloads as I
from tests.conftest import ROOT

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libbsr_attn.so not built")

SRC = os.path.join(ROOT, "block_sparse_paged_bsr_amd", "csrc", "kernels", "attn_prefill_bf16.hip")


def _kernel_constant(name):
    m = re.search(r"constexpr int %s = (\d+)[;,]" % name, open(SRC).read())
    assert m, name
    return int(m.group(1))


PAGE_WINDOW = _kernel_constant("kPageWindow")
TILE_KV = _kernel_constant("kTileKV")
BATCHES_PER_STEP = _kernel_constant("kDmaBatchesPerStep")
ISSUE_TO_USE = _kernel_constant("kIssueToUseSteps")  # steps between a tile's loads and its first read
K_AHEAD, V_AHEAD = ISSUE_TO_USE + 1, ISSUE_TO_USE - 1  # step j loads K(j + K_AHEAD), V(j + V_AHEAD)
MAX_IN_FLIGHT = BATCHES_PER_STEP * (ISSUE_TO_USE - 1)


def _page_no(t, kv_end, P):
    return np.minimum(t, kv_end - 1) // P


def window_states(kv_end, P, covers, fill_short=0):
    """Paging::cover over a sequence of (lo, hi) token ranges: the window's first page and its
    filled length after each call, and the number of refills after the first fill.
    (fill_short plants a mistake: a fill that stops that many entries early.)"""
    base, cnt, fills = -PAGE_WINDOW, 0, 0
    last = (kv_end - 1) // P
    bases, cnts = [], []
    for lo, hi in covers:
        plo, phi = min(lo, kv_end - 1) // P, min(hi, kv_end - 1) // P
        if not (plo >= base and phi < base + PAGE_WINDOW):
            base, cnt, fills = plo, min(PAGE_WINDOW, last - plo + 1) - fill_short, fills + 1
            assert phi - plo < cnt, "a cover() range wider than the window"
        bases.append(base)
        cnts.append(cnt)
    return np.array(bases), np.array(cnts), fills - 1


def check_lookups(first_tok, base, cnt, kv_end, P, span):
    """Table reads for tokens first_tok + 0 .. span-1 under windows (base, cnt), arrays over
    steps: the first and last token bound the index of every lane."""
    lo = _page_no(first_tok, kv_end, P) - base
    hi = _page_no(first_tok + span - 1, kv_end, P) - base
    assert lo.min() >= 0 and (hi - cnt).max() < 0, "a page id read outside the filled window"


@functools.lru_cache(maxsize=None)
def check_rings(n, n_full):
    return replay_rings(n, n_full)


def replay_rings(n, n_full, loose=0):
    """The DMA issue / wait / barrier / read sequence of one item of n 32-token tiles (n_full
    of them full; fast steps exist only where it is > 0).  Returns the number of fast steps.
    (loose plants a mistake: every wait lets that many more batches stay in flight.)"""
    queue = []  # batches of this wave not yet known complete, in issue order: (ring, tile)
    holds = {"K": {}, "V": {}}
    inflight = {"K": {}, "V": {}}
    last_read = {"K": {}, "V": {}}
    epoch = [0]
    issued = [0]

    def issue(ring, tile):
        assert 0 <= tile < n, f"DMA of nonexistent tile {ring}({tile})"
        slot = tile % 4
        assert last_read[ring].get(slot, -1) < epoch[0], f"{ring}({tile}) overwrites a slot read this step"
        assert slot not in inflight[ring], f"two loads in flight into {ring} slot {slot}"
        inflight[ring][slot] = tile
        queue.append((ring, tile))
        issued[0] += 1

    def wait(n_allowed):
        done = queue[: len(queue) - n_allowed] if n_allowed else list(queue)
        for ring, tile in done:
            assert inflight[ring].pop(tile % 4) == tile
            holds[ring][tile % 4] = tile
        del queue[: len(done)]

    def barrier():
        epoch[0] += 1
        issued[0] = 0

    def read(ring, tile, must_hold=True):
        slot = tile % 4
        assert slot not in inflight[ring], f"read of {ring} slot {slot} while a load fills it"
        if must_hold:
            assert holds[ring].get(slot) == tile, f"{ring}({tile}) not staged when read"
        last_read[ring][slot] = epoch[0]

    # prologue: K(0 .. K_AHEAD-1), V(0 .. V_AHEAD-1), then a full wait and a barrier; the first
    # scores read K(0)
    for t in range(K_AHEAD):
        if t < n:
            issue("K", t)
    for t in range(V_AHEAD):
        if t < n:
            issue("V", t)
    wait(0)
    barrier()
    read("K", 0)
    fast_steps = 0
    for j in range(n + 1):
        fast = j >= 1 and j + K_AHEAD + 1 < n_full
        # batches issued in the steps after the ones this step needs, that exist in the item
        nb = MAX_IN_FLIGHT if fast else sum((j - s + K_AHEAD < n) + (j - s + V_AHEAD < n)
                                            for s in range(1, ISSUE_TO_USE))
        assert nb <= MAX_IN_FLIGHT
        wait(nb + loose)
        barrier()
        if fast:
            fast_steps += 1
            issue("K", j + K_AHEAD)
            issue("V", j + V_AHEAD)
            assert issued[0] == BATCHES_PER_STEP
        else:
            if j + K_AHEAD < n:
                issue("K", j + K_AHEAD)
            if j + V_AHEAD < n:
                issue("V", j + V_AHEAD)
            assert issued[0] <= BATCHES_PER_STEP
        # the stream: scores of tile j+1 (masked out entirely when it does not exist), P.V of j-1
        read("K", j + 1, must_hold=j + 1 < n)
        read("V", 0 if j == 0 else j - 1)
    wait(0)
    return fast_steps


def model_pipelined(kv0, kv_end, P, div32, rings=True):
    """prefill_item128 and the pipelined prefill_item32: one 32-token tile per step, K loaded
    K_AHEAD tiles ahead and V V_AHEAD, lookups of K(j + K_AHEAD + 1) and V(j + V_AHEAD + 1) after
    cover(T(j + V_AHEAD + 1), T(j + K_AHEAD + 2) - 1).  Every lane of either shape loads one of a
    tile's 32 tokens.  Returns (refills, fast steps)."""
    n = (kv_end - kv0 + 31) // 32
    T = lambda j: kv0 + 32 * np.asarray(j)  # noqa: E731
    js = np.arange(n + 1)
    covers = [(kv0, kv0 + (K_AHEAD + 2) * 32 - 1)] + [(kv0 + 32 * (j + V_AHEAD + 1), kv0 + 32 * (j + K_AHEAD + 2) - 1)
                                                      for j in range(n + 1)]
    base, cnt, refills = window_states(kv_end, P, covers)
    # prologue lookups K(0 .. K_AHEAD), V(0 .. V_AHEAD) under the first window
    check_lookups(T(np.arange(K_AHEAD + 1)), base[0], cnt[0], kv_end, P, 32)
    # step j looks up K(j + K_AHEAD + 1) and V(j + V_AHEAD + 1) under the window after its cover()
    check_lookups(T(js + K_AHEAD + 1), base[1:], cnt[1:], kv_end, P, 32)
    check_lookups(T(js + V_AHEAD + 1), base[1:], cnt[1:], kv_end, P, 32)
    n_full = (kv_end - kv0) // 32 if div32 else 0
    fast = (js >= 1) & (js + K_AHEAD + 1 < n_full)
    if div32 and fast.any():
        # fast lookups: table[(kv0 + tok) / P + (j + ahead) (32 / P) - base], every token offset
        jf, tok = js[fast][:, None], np.arange(32)[None, :]
        bf, cf = base[1:][fast][:, None], cnt[1:][fast][:, None]
        for ahead in (K_AHEAD + 1, V_AHEAD + 1):
            idx = (kv0 + tok) // P + (jf + ahead) * (32 // P) - bf
            want = _page_no(kv0 + 32 * (jf + ahead) + tok, kv_end, P) - bf
            assert np.array_equal(idx, want) and idx.min() >= 0 and (idx - cf).max() < 0
        # and the row offset inside the page is the same in every tile
        assert np.array_equal((kv0 + 32 * jf + tok) % P, np.broadcast_to((kv0 + tok) % P, (len(jf), 32)))
    fast_steps = check_rings(n, n_full) if rings else int(fast.sum())
    return refills, fast_steps


def model_tile_loop(kv0, kv_end, P):
    """tile_loop of the smaller shapes: 64-token tiles in two stages; the four waves' lanes
    load tokens 0 .. 63 of a tile; every wait drains all loads.  Returns the refills."""
    ntiles = (kv_end - kv0 + TILE_KV - 1) // TILE_KV
    tis = np.arange(0, ntiles, 2)
    covers = [(kv0, kv0 + 2 * TILE_KV - 1)] + [(kv0 + (ti + 2) * TILE_KV, kv0 + (ti + 4) * TILE_KV - 1)
                                               for ti in tis]
    base, cnt, refills = window_states(kv_end, P, covers)
    check_lookups(np.array([kv0, kv0 + TILE_KV]), base[0], cnt[0], kv_end, P, TILE_KV)
    for ahead in (2, 3):
        check_lookups(kv0 + (tis + ahead) * TILE_KV, base[1:], cnt[1:], kv_end, P, TILE_KV)
    return refills


def _tables(kv_lens, P, seed, pool=None):
    """BSR arrays for requests of the given lengths, pages drawn from a random permutation of
    the pool (the layout of the workloads)."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    need = int(((kv_lens + P - 1) // P).sum())
    perm = np.random.default_rng(seed).permutation(pool or need)
    return I.page_table_from_lengths(kv_lens, P, perm)


def _run_plan(kv_lens, qo_indptr, P, C, causal, tile_q=0, shapes=("pipelined",), Hq=32, Hk=8, pool=None, seed=0,
              rings=True):
    ip, ix, last = _tables(kv_lens, P, seed, pool)
    p = api.Plan(ip, ix, last, num_pages=pool or max(len(ix), 1), num_qo_heads=Hq, num_kv_heads=Hk, head_dim=128,
                 page_size=P, qo_indptr=qo_indptr, causal=causal, num_workers=C, tile_q=tile_q)
    e = p.export()
    div32 = P <= 32 and (P & (P - 1)) == 0
    refills = fast = 0
    for it in e["items"]:
        kv_start, kv_len = int(it[4]), int(it[5])
        if "pipelined" in shapes:
            r, f = model_pipelined(kv_start, kv_start + kv_len, P, div32, rings)
            refills, fast = refills + r, fast + f
        if "loop" in shapes:
            refills += model_tile_loop(kv_start, kv_start + kv_len, P)
    return {"items": len(e["items"]), "refills": refills, "fast_steps": fast, "tile_q": int(e["tile_q"])}


def _qo(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def test_constants_agree_with_the_kernel():
    """The kernel derives its lookahead from kIssueToUseSteps in the same way as this model."""
    src = open(SRC).read()
    assert re.search(r"constexpr int kKAhead = kIssueToUseSteps \+ 1, kVAhead = kIssueToUseSteps - 1;", src)
    assert re.search(r"constexpr int kMaxBatchesInFlight = kDmaBatchesPerStep \* \(kIssueToUseSteps - 1\);", src)
    assert BATCHES_PER_STEP == 2 and ISSUE_TO_USE >= 2 and MAX_IN_FLIGHT <= 4


@pytest.mark.parametrize("n", range(1, 80))
def test_rings_every_short_item(n):
    """Every item length up to 80 tiles, with and without fast steps (n_full = n or n - 1)."""
    check_rings(n, 0)
    check_rings(n, n)
    check_rings(n, n - 1)


def test_ragged_causal_prefill_plan():
    """The batch-16 ragged causal prefill (page size 16) at 64 workers."""
    lens = I.prefill_lengths(0)
    r = _run_plan(lens, _qo(lens), 16, 64, True, shapes=("pipelined", "loop"))
    assert r["tile_q"] == 128 and r["fast_steps"] > 0


def test_vector_sparse_prefill_plan():
    """Batch 8 x 2048 causal prefill at page size 1 in a 2^20-row pool: items of up to 2048
    pages, exactly one full window."""
    lens = [2048] * 8
    r = _run_plan(lens, _qo(lens), 1, 64, True, shapes=("pipelined", "loop"), pool=1 << 20)
    assert r["refills"] == 0


def test_shared_prefix_level_plans():
    """The shared-prefix level of the batch-64 / 32,768-token shape: one block row of all 64
    queries, non-causal; chunked at 64 workers and as one 2048-page item per tile."""
    for C in (64, 1):
        r = _run_plan([32768], np.array([0, 64], dtype=np.int32), 16, C, False, shapes=("pipelined", "loop"))
        assert r["refills"] == 0


@pytest.mark.parametrize("P,L", [(1, 5000), (1, 2049), (16, 40000), (8, 17000), (12, 30000), (32, 70000)])
def test_items_longer_than_the_window(P, L):
    """Single causal requests whose work items span more than kPageWindow pages (mid-item
    window refills), for the pipelined shapes and the plain loop.  The ring accounting depends
    only on an item's tile count and is replayed in full above and for the shorter items here."""
    r = _run_plan([L], _qo([L]), P, 1, True, tile_q=128, shapes=("pipelined",), Hq=4, Hk=1, rings=L <= 6000)
    assert r["refills"] > 0
    for tq in (32, 64):
        r = _run_plan([L], _qo([L]), P, 1, True, tile_q=tq, shapes=("loop",), Hq=4, Hk=1)
        assert r["refills"] > 0


def test_model_catches_planted_mistakes():
    """The model is not vacuous: a wait one batch too loose, and a window fill one entry short,
    both fail it."""
    with pytest.raises(AssertionError, match="not staged|while a load fills it"):
        replay_rings(20, 20, loose=1)
    with pytest.raises(AssertionError, match="outside the filled window"):
        kv_end = 3000
        n = (kv_end + 31) // 32
        covers = [(0, 32 * (K_AHEAD + 2) - 1)] + [(32 * (j + V_AHEAD + 1), 32 * (j + K_AHEAD + 2) - 1)
                                                  for j in range(n + 1)]
        base, cnt, _ = window_states(kv_end, 1, covers, fill_short=1)
        js = np.arange(n + 1)
        check_lookups(32 * (js + K_AHEAD + 1), base[1:], cnt[1:], kv_end, 1, 32)


@pytest.mark.parametrize("tile_q", [128, 64, 32])
def test_page_window_refill_gpu_case(tile_q):
    """The exact plans of the GPU test of items longer than the window (5,000 tokens at page
    size 1, 8/2 heads, one worker), replayed here before they run on the GPU."""
    r = _run_plan([5000], _qo([5000]), 1, 1, True, tile_q=tile_q, shapes=("pipelined", "loop"), Hq=8, Hk=2,
                  pool=5300, seed=11)
    assert r["refills"] > 0


# ---- steady steps: the straight-line steps of the pipelined shapes ----
# The kernels run a subset of an item's steps as straight-line code (four per loop trip, LDS
# slots fixed at compile time, a fixed wait, no window test and, without VAR in the 128-row
# shape, no mask).  The bounds below are the kernels' (C++ integer division truncates toward
# zero); the checks are the conditions under which those steps may skip the tests.

def _trunc_div(a, b):
    q = abs(a) // b
    return q if a >= 0 else -q


def steady_steps(kv0, kv_end, min_lim, window_holds, div32, max_lo=None, mask_every_step=False, hi_slack=0):
    """Steps j of one item that run as steady steps: from j_fast (a multiple of 4) n_quads
    quads.  max_lo: the sliding window's largest lower bound over the tile's rows (128-row shape
    with VAR); mask_every_step: the 4-wave shape with VAR, whose steady steps apply the mask.
    (hi_slack plants a mistake: a last steady step that many steps too late.)"""
    if not (div32 and window_holds):
        return []
    n_full = (kv_end - kv0) // 32
    hi = n_full - K_AHEAD - 2 + hi_slack
    if not mask_every_step:
        hi = min(hi, _trunc_div(min_lim - kv0, 32) - 2 + hi_slack)
    lo = 1
    if max_lo is not None and max_lo > kv0:
        lo = max(lo, (max_lo - kv0 + 31) // 32 - 1)
    lo = (lo + 3) & ~3
    if hi < lo:
        return []
    return list(range(lo, lo + 4 * ((hi - lo + 1) // 4)))


def check_steady(kv0, kv_end, min_lim, steps, max_lo=None, mask_every_step=False):
    n = (kv_end - kv0 + 31) // 32
    n_full = (kv_end - kv0) // 32
    for j in steps:
        assert 1 <= j <= n, "a steady step outside the item"
        # the model's fast-step condition: lookups and loads of full tiles of the fast page class
        assert j + K_AHEAD + 1 < n_full, f"steady step {j} of {n_full} full tiles loads a partial tile"
        t1 = kv0 + 32 * (j + 1)  # first key of the score tile the step computes
        if not mask_every_step:
            assert t1 + 32 <= min_lim, f"steady step {j} skips the causal mask of tile {j + 1}"
            if max_lo is not None:
                assert t1 >= max_lo, f"steady step {j} skips the window mask of tile {j + 1}"
    assert steps == sorted(steps) and (not steps or steps[0] % 4 == 0), "steady steps start at a multiple of 4"
    assert len(steps) % 4 == 0


def _steady_over_plan(kv_lens, qo_lens, P, C, causal, window_left=-1, shape="128", hi_slack=0, pool=None):
    ip, ix, last = _tables(kv_lens, P, 0, pool)
    qo = _qo(qo_lens)
    p = api.Plan(ip, ix, last, num_pages=pool or max(len(ix), 1), num_qo_heads=32, num_kv_heads=8, head_dim=128,
                 page_size=P, qo_indptr=qo, causal=causal, num_workers=C, tile_q=128, window_left=window_left)
    e = p.export()
    g = 4
    div32 = P <= 32 and (P & (P - 1)) == 0
    total = 0
    for it in e["items"]:
        req, r0, r1, kv0, kl = int(it[0]), int(it[2]), int(it[3]), int(it[4]), int(it[5])
        kv_end = kv0 + kl
        lq, lk = int(qo[req + 1] - qo[req]), int(kv_lens[req])
        min_lim = min(kv_end, lk - lq + r0 // g + 1) if causal else kv_end
        window_holds = _page_no(kv_end - 1, kv_end, P) - _page_no(kv0, kv_end, P) < PAGE_WINDOW
        max_lo = (lk - lq - window_left + (r1 - 1) // g) if window_left >= 0 else None
        var = window_left >= 0
        if shape == "128":
            steps = steady_steps(kv0, kv_end, min_lim, window_holds, div32, max_lo if var else None,
                                 hi_slack=hi_slack)
            check_steady(kv0, kv_end, min_lim, steps, max_lo if var else None)
        else:  # the 4-wave shape (128-row tiles of soft-capped plans): with VAR the mask runs in every step
            steps = steady_steps(kv0, kv_end, min_lim, window_holds, div32, mask_every_step=var, hi_slack=hi_slack)
            check_steady(kv0, kv_end, min_lim, steps, mask_every_step=var)
        total += len(steps)
    return total


@pytest.mark.parametrize("shape", ["128", "32"])
def test_steady_steps_ragged_and_uniform_plans(shape):
    """The ragged causal prefill and uniform batches (causal and not), page sizes 16 and 1."""
    lens = I.prefill_lengths(0)
    assert _steady_over_plan(lens, lens, 16, 64, True, shape=shape) > 0
    assert _steady_over_plan([4096] * 4, [4096] * 4, 16, 64, True, shape=shape) > 0
    assert _steady_over_plan([3000, 700, 45], [3000, 700, 45], 1, 16, False, shape=shape, pool=1 << 14) > 0
    assert _steady_over_plan([2048] * 2, [300, 2048], 8, 8, True, shape=shape) > 0


@pytest.mark.parametrize("shape", ["128", "32"])
def test_steady_steps_sliding_window(shape):
    """Windowed causal prefill (the VAR instantiations): windows of 1024 and 100 keys."""
    lens = I.prefill_lengths(0)
    for w in (1023, 99):
        _steady_over_plan(lens, lens, 16, 64, True, window_left=w, shape=shape)


def test_steady_steps_planted_mistake():
    """A last steady step one step too late is caught (it would load a partial tile or skip a
    mask)."""
    lens = I.prefill_lengths(0)
    with pytest.raises(AssertionError, match="partial tile|skips the"):
        _steady_over_plan(lens, lens, 16, 64, True, hi_slack=1)
