// Host planner of composable formats: attention over the union of several BSR views of one KV
// pool, the views' attention states combined with the merge operator.
//
// "FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for LLM Inference
// Serving" §IV.6 and "FlashInfer 原理" §⑤: a batch whose requests share a prefix is stored as
// several block-sparse matrices -- the shared prefix as a block row of several queries (B_r > 1),
// the private suffixes at B_r = 1 -- and each query's attention over its whole context is the ⊕ of
// its states over the views (eq. 6 of "FlashInfer: Making Attention Fit the Serving Workload"; its
// §7.3 and eq. 15 give the traffic saved: a shared block is read once per block row).
//
// Plan: every view's block rows are cut into query tiles of 16 packed rows (so that the decode
// kernel's 16 matrix columns serve a tile, and a shared block row of 4 queries x 4 heads is one
// tile), and the tiles of all views are scheduled together by the same longest-processing-time
// partition as a single view (total work over all views, one chunk limit, one stable sort, one
// heap): one attention launch then covers every view.  Every chunk writes a partial state; the
// reduction map has one entry per query, listing that query's partial rows in every view (views in
// order, chunks in KV order), so one merge pass folds the views and the chunks together.
#include <algorithm>
#include <cstring>
#include <functional>
#include <numeric>
#include <queue>
#include <sstream>
#include <utility>

#include "bsr_internal.h"

namespace bsr {

namespace {

constexpr int32_t kComposeTile = 16;  // packed rows per query tile in a composable plan
constexpr int32_t kMaxLevels = 16;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

int cfail(const std::string& m) {
  set_error(m);
  return BSR_INVALID_ARG;
}

}  // namespace

int build_composable_plan(const bsr_plan_desc* levels, int32_t n_levels, int32_t num_workers, bsr_plan* p) {
  if (!levels) return cfail("levels is NULL");
  if (n_levels < 1 || n_levels > kMaxLevels) return cfail("n_levels must be 1 .. 16");
  if (num_workers < 0) return cfail("num_workers must be >= 0");
  const bsr_plan_desc& d0 = levels[0];
  std::vector<bsr_plan> lv(n_levels);
  int32_t total_q = -1;
  for (int32_t l = 0; l < n_levels; ++l) {
    const bsr_plan_desc& d = levels[l];
    if (d.num_qo_heads != d0.num_qo_heads || d.num_kv_heads != d0.num_kv_heads || d.head_dim != d0.head_dim ||
        d.page_size != d0.page_size || d.num_pages != d0.num_pages)
      return cfail("every level must share num_qo_heads, num_kv_heads, head_dim, page_size and num_pages");
    if (d.causal) return cfail("composable levels are non-causal (a level's keys are all visible to its queries)");
    if (d.window_size != 0) return cfail("composable levels take no sliding window");
    if (d.logits_soft_cap != d0.logits_soft_cap) return cfail("every level must share logits_soft_cap");
    if (d.alpha != d0.alpha || d.beta != d0.beta) return cfail("every level must share alpha and beta");
    bsr_plan_desc dd = d;
    dd.tile_q = kComposeTile;
    dd.num_workers = 1;  // the per-level schedule is not used; the levels are scheduled together
    std::ostringstream pre;
    const int rc = build_plan(&dd, &lv[l]);
    if (rc != BSR_OK) {
      pre << "level " << l << ": ";
      return cfail(pre.str() + bsr_last_error());
    }
    const int32_t nq = lv[l].qo_indptr[lv[l].B];
    if (total_q < 0) total_q = nq;
    if (nq != total_q) return cfail("every level must hold the same queries (equal qo_indptr[B] / batch)");
  }
  const int32_t g = lv[0].g;
  if (kComposeTile % g != 0) return cfail("composable plans need a group size that divides 16 (1, 2, 4, 8, 16)");

  p->B = 0;
  for (const auto& x : lv) p->B += x.B;
  p->Hq = lv[0].Hq;
  p->Hk = lv[0].Hk;
  p->g = g;
  p->d = lv[0].d;
  p->P = lv[0].P;
  p->causal = 0;
  p->C = num_workers ? num_workers : 256;
  p->alpha = lv[0].alpha;
  p->beta = lv[0].beta;
  p->num_pages = lv[0].num_pages;
  p->window_left = -1;
  p->soft_cap = lv[0].soft_cap;
  p->decode = false;
  p->Tq = kComposeTile;
  p->num_levels = n_levels;

  // ---- flattened requests: the levels' block rows, level after level ----
  p->level_req_start.assign(n_levels + 1, 0);
  p->qo_indptr.clear();
  p->kv_indptr.assign(1, 0);
  p->kv_indices.clear();
  p->last_page_len.clear();
  p->qo_len.clear();
  p->kv_len.clear();
  p->total_kv_tokens = 0;
  p->max_qo_len = 0;
  std::vector<int32_t> q_start;  // first query of each flattened request
  for (int32_t l = 0; l < n_levels; ++l) {
    const bsr_plan& x = lv[l];
    p->level_req_start[l] = int32_t(p->kv_len.size());
    const int32_t base = int32_t(p->kv_indices.size());
    for (int32_t i = 0; i < x.B; ++i) {
      q_start.push_back(x.qo_indptr[i]);
      p->qo_len.push_back(x.qo_len[i]);
      p->kv_len.push_back(x.kv_len[i]);
      p->last_page_len.push_back(x.last_page_len[i]);
      p->kv_indptr.push_back(base + x.kv_indptr[i + 1]);
      p->max_qo_len = std::max(p->max_qo_len, x.qo_len[i]);
    }
    p->kv_indices.insert(p->kv_indices.end(), x.kv_indices.begin(), x.kv_indices.end());
    p->total_kv_tokens += x.total_kv_tokens;
  }
  p->level_req_start[n_levels] = p->B;
  if (p->total_kv_tokens > INT32_MAX) return cfail("total KV tokens exceed int32");
  p->qo_indptr = q_start;  // (per flattened request: its first query)
  p->qo_indptr.push_back(total_q);
  p->mask_bits = 0;

  // ---- tiles of every level (16 packed rows, non-causal: the whole KV row is visible) ----
  p->tiles.clear();
  p->tile_lo.clear();
  std::vector<int32_t> tile_first(p->B + 1, 0);  // first tile of each flattened request
  int64_t W = 0;
  for (int32_t l = 0; l < n_levels; ++l) {
    const bsr_plan& x = lv[l];
    const int32_t r0 = p->level_req_start[l];
    for (int32_t t = 0; t < int32_t(x.tiles.size() / 5); ++t) {
      const int32_t* tr = &x.tiles[5 * t];
      if (t == 0 || x.tiles[5 * (t - 1)] != tr[0]) tile_first[r0 + tr[0]] = int32_t(p->tiles.size() / 5);
      p->tiles.insert(p->tiles.end(), {r0 + tr[0], tr[1], tr[2], tr[3], 0});
      p->tile_lo.push_back(0);
    }
    W += x.W;  // eq. 10 per level; the levels' sum is the batch's total work
  }
  const int32_t num_tiles = int32_t(p->tiles.size() / 5);
  p->W = W;
  p->L = (W > 0) ? std::max<int64_t>(1, cdiv(W, p->C)) : 0;

  // ---- chunks (creation order: level, request, tile, kv_start), longest first, least loaded ----
  struct Item {
    int32_t req, tile, r0, r1, ks, kl, worker, slot;
  };
  std::vector<Item> items;
  std::vector<std::vector<int32_t>> tile_items(num_tiles);
  if (p->L > 0)
    for (int32_t t = 0; t < num_tiles; ++t) {
      const int32_t* tr = &p->tiles[5 * t];
      for (int64_t s = 0; s < tr[3]; s += p->L) {
        tile_items[t].push_back(int32_t(items.size()));
        items.push_back({tr[0], t, tr[1], tr[2], int32_t(s), int32_t(std::min<int64_t>(p->L, tr[3] - s)), -1, -1});
      }
      p->tiles[5 * t + 4] = int32_t(tile_items[t].size());
    }
  const int32_t M = int32_t(items.size());
  std::vector<int32_t> order(M);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return items[a].kl > items[b].kl; });
  using Key = std::pair<int64_t, int32_t>;
  std::priority_queue<Key, std::vector<Key>, std::greater<Key>> heap;
  for (int32_t w = 0; w < p->C; ++w) heap.push({0, w});
  std::vector<std::vector<int32_t>> queues(p->C);
  p->worker_cost.assign(p->C, 0);
  for (int32_t m : order) {
    Key k = heap.top();
    heap.pop();
    queues[k.second].push_back(m);
    items[m].worker = k.second;
    const int64_t positions = (items[m].r1 - 1) / g - items[m].r0 / g + 1;
    k.first += int64_t(p->alpha) * positions + int64_t(p->beta) * items[m].kl;
    p->worker_cost[k.second] = k.first;
    heap.push(k);
  }
  // every chunk writes a partial state (the views are folded by the merge pass), slots in
  // assignment order
  int32_t slot = 0;
  for (int32_t m : order) items[m].slot = slot++;
  p->num_slots = slot;

  // ---- reduction map: one entry per query; its rows in every level, levels in order, chunks in
  // KV order ----
  p->merge_tiles.clear();
  p->merge_ptr.assign(1, 0);
  p->merge_slots.clear();
  p->merge_roff.clear();
  for (int32_t q = 0; q < total_q; ++q) {
    for (int32_t l = 0; l < n_levels; ++l) {
      const bsr_plan& x = lv[l];
      // the level's block row holding query q (qo_indptr is non-decreasing; empty rows skipped)
      const int32_t i = int32_t(std::upper_bound(x.qo_indptr.begin(), x.qo_indptr.end(), q) - x.qo_indptr.begin()) - 1;
      const int32_t fr = p->level_req_start[l] + i;
      const int32_t row = (q - x.qo_indptr[i]) * g;
      const int32_t t = tile_first[fr] + row / kComposeTile;
      for (int32_t m : tile_items[t]) {
        p->merge_slots.push_back(items[m].slot);
        p->merge_roff.push_back(row - p->tiles[5 * t + 1]);
      }
    }
    p->merge_tiles.push_back(q);
    p->merge_ptr.push_back(int32_t(p->merge_slots.size()));
  }

  // ---- exported arrays ----
  p->items.resize(size_t(M) * 8);
  for (int32_t m = 0; m < M; ++m) {
    const Item& it = items[m];
    int32_t* r = &p->items[size_t(m) * 8];
    r[0] = it.req; r[1] = it.tile; r[2] = it.r0; r[3] = it.r1;
    r[4] = it.ks; r[5] = it.kl; r[6] = it.worker; r[7] = it.slot;
  }
  p->queue_ptr.assign(p->C + 1, 0);
  p->queue_items.clear();
  for (int32_t w = 0; w < p->C; ++w) {
    p->queue_items.insert(p->queue_items.end(), queues[w].begin(), queues[w].end());
    p->queue_ptr[w + 1] = int32_t(p->queue_items.size());
  }

  // ---- workspace layout and the metadata image ----
  WsLayout& L = p->ws;
  const int64_t nnz = int64_t(p->kv_indices.size());
  const int32_t NM = int32_t(p->merge_tiles.size());
  size_t off = 0;
  L.req = off;      off = al256(off + sizeof(ReqRec) * std::max(p->B, 1));
  L.indices = off;  off = al256(off + sizeof(int32_t) * std::max<int64_t>(nnz, 1));
  L.items = off;    off = al256(off + sizeof(ItemRec) * std::max(M, 1));
  L.qptr = off;     off = al256(off + sizeof(int32_t) * (p->C + 1));
  L.merge = off;    off = al256(off + sizeof(MergeRec) * std::max(NM, 1));
  L.mslots = off;   off = al256(off + sizeof(int32_t) * std::max<size_t>(p->merge_slots.size(), 1));
  L.mroff = off;    off = al256(off + sizeof(int32_t) * std::max<size_t>(p->merge_roff.size(), 1));
  L.lpt = off;      off = al256(off + sizeof(int32_t) * std::max(M, 1));
  L.items_lpt = off; off = al256(off + sizeof(ItemRec) * std::max(M, 1));
  L.tickets = off;  off = al256(off + sizeof(int32_t) * 2 * kTicketGroups);
  // (a query's states span several tiles: the merge pass folds them, never the attention kernel)
  L.imerge = off;   off = al256(off + sizeof(int32_t) * std::max(M, 1));
  L.arrive = off;   off = al256(off + sizeof(int32_t));
  L.meta_bytes = off;
  const size_t rows_per_slot = size_t(p->Hk) * p->Tq;
  L.part_o = off;   off = al256(off + sizeof(float) * rows_per_slot * p->d * p->num_slots);
  L.part_lse = off; off = al256(off + sizeof(float) * rows_per_slot * p->num_slots);
  L.total = off;
  p->meta.assign(L.meta_bytes, 0);
  {
    auto* im = reinterpret_cast<int32_t*>(p->meta.data() + L.imerge);
    std::fill(im, im + std::max(M, 1), -1);
    p->item_folds = false;
  }
  auto* req = reinterpret_cast<ReqRec*>(p->meta.data() + L.req);
  int64_t tok = 0;
  for (int32_t i = 0; i < p->B; ++i) {
    req[i].q_start = q_start[i];
    req[i].q_len = p->qo_len[i];
    req[i].page_start = p->kv_indptr[i];
    req[i].kv_len = p->kv_len[i];
    req[i].tok_start = int32_t(tok);
    req[i].mask_off = 0;
    tok += p->kv_len[i];
  }
  if (nnz > 0) std::memcpy(p->meta.data() + L.indices, p->kv_indices.data(), sizeof(int32_t) * nnz);
  auto* qi = reinterpret_cast<ItemRec*>(p->meta.data() + L.items);
  for (int32_t k = 0; k < M; ++k) {
    const Item& it = items[p->queue_items[k]];
    qi[k] = ItemRec{it.req, it.r0, it.r1, it.ks, it.ks + it.kl, it.slot, req[it.req].q_start, req[it.req].page_start,
                    req[it.req].q_len, req[it.req].kv_len, {0, 0, 0, 0}};
  }
  std::memcpy(p->meta.data() + L.qptr, p->queue_ptr.data(), sizeof(int32_t) * (p->C + 1));
  // the items in the partition's LPT order (longest first), as positions in the queue-ordered list
  {
    std::vector<int32_t> pos(M);
    for (int32_t k = 0; k < M; ++k) pos[p->queue_items[k]] = k;
    auto* lpt = reinterpret_cast<int32_t*>(p->meta.data() + L.lpt);
    for (int32_t t = 0; t < M; ++t) lpt[t] = pos[order[t]];
    // the records in that order (no merge records: the merge pass folds composable plans)
    auto* ql = reinterpret_cast<ItemRec*>(p->meta.data() + L.items_lpt);
    for (int32_t t = 0; t < M; ++t) {
      ql[t] = qi[lpt[t]];
      ql[t].pad[0] = -1;
    }
  }
  auto* mr = reinterpret_cast<MergeRec*>(p->meta.data() + L.merge);
  for (int32_t k = 0; k < NM; ++k)
    mr[k] = MergeRec{p->merge_tiles[k], 0, g, p->merge_ptr[k], p->merge_ptr[k + 1] - p->merge_ptr[k], 1, {0, 0}};
  if (!p->merge_slots.empty()) {
    std::memcpy(p->meta.data() + L.mslots, p->merge_slots.data(), sizeof(int32_t) * p->merge_slots.size());
    std::memcpy(p->meta.data() + L.mroff, p->merge_roff.data(), sizeof(int32_t) * p->merge_roff.size());
  }
  return BSR_OK;
}

}  // namespace bsr
