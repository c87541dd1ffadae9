// Host planner: validation, the longest-processing-time split-KV partition and the
// device image of the plan (work queues + reduction map at fixed workspace offsets).
//
// The partition follows FlashInfer's runtime scheduler as described in
// "FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for LLM
// Inference Serving" (§VIII.2-VIII.5), "FlashInfer 原理" (§⑦, §⑨) and
// "FlashInfer: Making Attention Fit the Serving Workload" (§6.1-6.2, eqs. 10-11).
// All costs are integers and every ordering decision is explicit (stable sort,
// lexicographic heap keys), so identical lengths give a byte-identical plan.
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

constexpr int32_t kTileSet[] = {16, 32, 64, 128};
constexpr int32_t kDefaultWorkers = 256;  // one per compute unit of an MI355X

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int fail(const std::string& m) {
  set_error(m);
  return BSR_INVALID_ARG;
}

}  // namespace

int build_plan(const bsr_plan_desc* desc, bsr_plan* p) {
  if (!desc) return fail("bsr_plan_create: desc is NULL");
  const int32_t B = desc->batch;
  if (B < 0) return fail("batch must be >= 0");
  if (desc->num_kv_heads < 1 || desc->num_qo_heads < 1)
    return fail("head counts must be >= 1");
  if (desc->num_qo_heads % desc->num_kv_heads != 0)
    return fail("num_qo_heads must be a multiple of num_kv_heads");
  if (desc->head_dim < 1) return fail("head_dim must be >= 1");
  if (desc->page_size < 1) return fail("page_size must be >= 1");
  if (int64_t(desc->page_size) * desc->num_kv_heads * desc->head_dim >= (int64_t(1) << 31))
    return fail("page_size * num_kv_heads * head_dim must be below 2^31 (elements of one page)");
  if (desc->num_workers < 0) return fail("num_workers must be >= 0");
  if (desc->tile_q < 0 || (desc->tile_q > 0 && desc->tile_q % 16 != 0) || desc->tile_q > 128)
    return fail("tile_q must be 0 or a multiple of 16 up to 128");
  if (desc->alpha < 0 || desc->beta < 0) return fail("alpha and beta must be >= 0");
  if (desc->num_pages < 0) return fail("num_pages must be >= 0");
  if (desc->window_size < 0) return fail("window_size must be 0 (no window) or >= 1");
  if (!(desc->logits_soft_cap >= 0.f) || desc->logits_soft_cap == __builtin_huge_valf())
    return fail("logits_soft_cap must be 0 (off) or positive and finite");
  if (B > 0 && (!desc->kv_indptr || !desc->last_page_len))
    return fail("kv_indptr and last_page_len are required");

  p->B = B;
  p->Hq = desc->num_qo_heads;
  p->Hk = desc->num_kv_heads;
  p->g = p->Hq / p->Hk;
  p->d = desc->head_dim;
  p->P = desc->page_size;
  p->causal = desc->causal ? 1 : 0;
  p->C = desc->num_workers ? desc->num_workers : std::max(1, kDefaultWorkers);
  p->alpha = desc->alpha;
  p->beta = desc->beta;
  if (p->alpha == 0 && p->beta == 0) {
    p->alpha = 2;
    p->beta = 1;
  }
  p->num_pages = desc->num_pages;
  p->window_left = desc->window_size - 1;  // keys left of the diagonal, -1 = no window
  p->soft_cap = desc->logits_soft_cap;
  p->decode = desc->qo_indptr == nullptr;

  // ---- copy and validate the BSR arrays ----
  p->kv_indptr.assign(B + 1, 0);
  if (B > 0) std::memcpy(p->kv_indptr.data(), desc->kv_indptr, sizeof(int32_t) * (B + 1));
  if (p->kv_indptr[0] != 0) return fail("kv_indptr[0] must be 0");
  for (int32_t i = 0; i < B; ++i)
    if (p->kv_indptr[i + 1] < p->kv_indptr[i]) return fail("kv_indptr must be non-decreasing");
  const int64_t nnz = p->kv_indptr[B];
  // kv_indices == NULL: contiguous KV, request i's pages are kv_indptr[i] .. kv_indptr[i+1] - 1 of
  // the pool in order (the identity table, stored like any other so that every kernel reads it)
  p->affine = desc->kv_indices == nullptr;
  p->kv_indices.assign(nnz, 0);
  if (p->affine) {
    for (int64_t k = 0; k < nnz; ++k) p->kv_indices[k] = int32_t(k);
  } else if (nnz > 0) {
    std::memcpy(p->kv_indices.data(), desc->kv_indices, sizeof(int32_t) * nnz);
  }
  for (int64_t k = 0; k < nnz; ++k)
    if (p->kv_indices[k] < 0 || p->kv_indices[k] >= p->num_pages) {
      std::ostringstream os;
      os << "kv_indices[" << k << "] = " << p->kv_indices[k] << " outside [0, " << p->num_pages
         << ")";
      return fail(os.str());
    }
  p->last_page_len.assign(B, 0);
  if (B > 0) std::memcpy(p->last_page_len.data(), desc->last_page_len, sizeof(int32_t) * B);
  p->kv_len.assign(B, 0);
  int64_t tok = 0;
  for (int32_t i = 0; i < B; ++i) {
    const int32_t n = p->kv_indptr[i + 1] - p->kv_indptr[i];
    const int32_t last = p->last_page_len[i];
    if (n > 0 && (last < 1 || last > p->P)) {
      std::ostringstream os;
      os << "last_page_len[" << i << "] = " << last << " outside [1, " << p->P << "]";
      return fail(os.str());
    }
    if (n == 0 && last != 0) return fail("last_page_len must be 0 for a request without pages");
    const int64_t l = n > 0 ? int64_t(n - 1) * p->P + last : 0;
    if (l > INT32_MAX / 2) return fail("KV length too large");
    p->kv_len[i] = int32_t(l);
    tok += l;
  }
  if (tok > INT32_MAX) return fail("total KV tokens exceed int32");
  p->total_kv_tokens = tok;

  p->qo_indptr.assign(B + 1, 0);
  p->qo_len.assign(B, 1);
  if (p->decode) {
    for (int32_t i = 0; i <= B; ++i) p->qo_indptr[i] = i;
  } else {
    std::memcpy(p->qo_indptr.data(), desc->qo_indptr, sizeof(int32_t) * (B + 1));
    if (p->qo_indptr[0] != 0) return fail("qo_indptr[0] must be 0");
    for (int32_t i = 0; i < B; ++i) {
      if (p->qo_indptr[i + 1] < p->qo_indptr[i]) return fail("qo_indptr must be non-decreasing");
      p->qo_len[i] = p->qo_indptr[i + 1] - p->qo_indptr[i];
    }
  }
  p->max_qo_len = 0;
  for (int32_t i = 0; i < B; ++i) p->max_qo_len = std::max(p->max_qo_len, p->qo_len[i]);
  if (int64_t(p->max_qo_len) * p->g > INT32_MAX / 2) return fail("query length too large");

  // ---- query tile: smallest of the tile set >= average packed query length ----
  std::vector<int64_t> pq(B);
  int64_t pq_sum = 0;
  for (int32_t i = 0; i < B; ++i) {
    pq[i] = int64_t(p->qo_len[i]) * p->g;
    pq_sum += pq[i];
  }
  if (desc->tile_q) {
    p->Tq = desc->tile_q;
  } else {
    const int64_t avg = B ? ceil_div(pq_sum, B) : 0;
    p->Tq = kTileSet[3];
    for (int32_t t : kTileSet)
      if (t >= avg) {
        p->Tq = t;
        break;
      }
  }
  const int32_t Tq = p->Tq;

  // ---- query tiles and their visible KV ranges ----
  // A tile sees keys [lo, vis): vis ends at the causal limit of its last query position;
  // with a sliding window of w keys to the left, lo is the window start of its first
  // query position ("FlashInfer 原理" §⑧: key k is visible to query q of a request iff
  // k + l_qo + w >= l_kv + q), clipped to [0, vis].
  p->tiles.clear();
  p->tile_lo.clear();
  for (int32_t i = 0; i < B; ++i) {
    const int64_t nt = ceil_div(pq[i], Tq);
    for (int64_t j = 0; j < nt; ++j) {
      const int64_t r0 = j * Tq, r1 = std::min<int64_t>(r0 + Tq, pq[i]);
      const int64_t last_pos = (r1 - 1) / p->g;
      int64_t vis = p->kv_len[i];
      if (p->causal)
        vis = std::max<int64_t>(0, std::min<int64_t>(p->kv_len[i],
                                                     int64_t(p->kv_len[i]) - p->qo_len[i] + last_pos + 1));
      int64_t lo = 0;
      if (p->window_left >= 0)
        lo = std::min<int64_t>(vis, std::max<int64_t>(0, int64_t(p->kv_len[i]) - p->qo_len[i] + r0 / p->g -
                                                             p->window_left));
      p->tiles.insert(p->tiles.end(), {i, int32_t(r0), int32_t(r1), int32_t(vis), 0});
      p->tile_lo.push_back(int32_t(lo));
    }
  }
  const int32_t num_tiles = int32_t(p->tiles.size() / 5);

  // ---- total work (eq. 10; with a window, the sum of the tiles' windowed ranges) and
  // chunk limit ----
  int64_t W = 0;
  if (p->window_left >= 0) {
    for (int32_t t = 0; t < num_tiles; ++t) W += p->tiles[5 * t + 3] - p->tile_lo[t];
  } else {
    for (int32_t i = 0; i < B; ++i) W += ceil_div(pq[i], Tq) * p->kv_len[i];
  }
  p->W = W;
  p->L = (B > 0 && W > 0) ? std::max<int64_t>(1, ceil_div(W, p->C)) : 0;

  // ---- work items: chunks in creation order ----
  struct Item {
    int32_t req, tile, r0, r1, ks, kl, worker, slot;
  };
  std::vector<Item> items;
  std::vector<std::vector<int32_t>> tile_items(num_tiles);
  if (p->L > 0) {
    for (int32_t t = 0; t < num_tiles; ++t) {
      const int32_t* tr = &p->tiles[5 * t];
      for (int64_t s = p->tile_lo[t]; s < tr[3]; s += p->L) {
        const int32_t n = int32_t(std::min<int64_t>(p->L, tr[3] - s));
        tile_items[t].push_back(int32_t(items.size()));
        items.push_back({tr[0], t, tr[1], tr[2], int32_t(s), n, -1, -1});
      }
      p->tiles[5 * t + 4] = int32_t(tile_items[t].size());
    }
  }
  const int32_t M = int32_t(items.size());

  // ---- longest first (stable: equal lengths keep creation order) ----
  std::vector<int32_t> order(M);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return items[a].kl > items[b].kl; });

  // ---- least-loaded worker first; ties go to the lower worker id ----
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
    // the item's query length: positions covered by its tile's packed rows
    const int64_t positions = (items[m].r1 - 1) / p->g - items[m].r0 / p->g + 1;
    k.first += int64_t(p->alpha) * positions + int64_t(p->beta) * items[m].kl;
    p->worker_cost[k.second] = k.first;
    heap.push(k);
  }

  // ---- partial slots for chunks of split tiles, in assignment order ----
  int32_t slot = 0;
  for (int32_t m : order)
    if (tile_items[items[m].tile].size() > 1) items[m].slot = slot++;
  p->num_slots = slot;

  // ---- reduction map: split and empty tiles, slots by ascending kv_start ----
  p->merge_tiles.clear();
  p->merge_ptr.assign(1, 0);
  p->merge_slots.clear();
  for (int32_t t = 0; t < num_tiles; ++t) {
    if (tile_items[t].size() == 1) continue;
    p->merge_tiles.push_back(t);
    // creation order already has ascending kv_start within a tile
    for (int32_t m : tile_items[t]) p->merge_slots.push_back(items[m].slot);
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
  size_t off = 0;
  L.req = off;      off = align256(off + sizeof(ReqRec) * std::max(B, 1));
  L.indices = off;  off = align256(off + sizeof(int32_t) * std::max<int64_t>(nnz, 1));
  L.items = off;    off = align256(off + sizeof(ItemRec) * std::max(M, 1));
  L.qptr = off;     off = align256(off + sizeof(int32_t) * (p->C + 1));
  const int32_t NM = int32_t(p->merge_tiles.size());
  L.merge = off;    off = align256(off + sizeof(MergeRec) * std::max(NM, 1));
  L.mslots = off;   off = align256(off + sizeof(int32_t) * std::max<size_t>(p->merge_slots.size(), 1));
  L.mroff = off;    off = align256(off + sizeof(int32_t));  // (no row offsets in a single-level plan)
  L.lpt = off;      off = align256(off + sizeof(int32_t) * std::max(M, 1));
  L.items_lpt = off; off = align256(off + sizeof(ItemRec) * std::max(M, 1));
  L.tickets = off;  off = align256(off + sizeof(int32_t) * 2 * kTicketGroups);
  L.imerge = off;   off = align256(off + sizeof(int32_t) * std::max(M, 1));
  L.arrive = off;   off = align256(off + sizeof(int32_t) * std::max<int64_t>(int64_t(NM) * p->Hk, 1));
  L.meta_bytes = off;
  const size_t rows_per_slot = size_t(p->Hk) * Tq;
  L.part_o = off;   off = align256(off + sizeof(float) * rows_per_slot * p->d * p->num_slots);
  L.part_lse = off; off = align256(off + sizeof(float) * rows_per_slot * p->num_slots);
  L.total = off;

  p->meta.assign(L.meta_bytes, 0);
  auto* req = reinterpret_cast<ReqRec*>(p->meta.data() + L.req);
  int64_t tok_start = 0, mask_off = 0;
  for (int32_t i = 0; i < B; ++i) {
    req[i].q_start = p->qo_indptr[i];
    req[i].q_len = p->qo_len[i];
    req[i].page_start = p->kv_indptr[i];
    req[i].kv_len = p->kv_len[i];
    req[i].tok_start = int32_t(tok_start);
    req[i].mask_off = mask_off;
    tok_start += p->kv_len[i];
    mask_off += int64_t(p->qo_len[i]) * p->kv_len[i];
  }
  p->mask_bits = mask_off;
  if (nnz > 0)
    std::memcpy(p->meta.data() + L.indices, p->kv_indices.data(), sizeof(int32_t) * nnz);
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
  }
  auto* mr = reinterpret_cast<MergeRec*>(p->meta.data() + L.merge);
  for (int32_t k = 0; k < NM; ++k) {
    const int32_t* tr = &p->tiles[5 * p->merge_tiles[k]];
    mr[k] = MergeRec{p->qo_indptr[tr[0]], tr[1], tr[2], p->merge_ptr[k], p->merge_ptr[k + 1] - p->merge_ptr[k], 0, {0, 0}};
  }
  if (!p->merge_slots.empty())
    std::memcpy(p->meta.data() + L.mslots, p->merge_slots.data(),
                sizeof(int32_t) * p->merge_slots.size());
  // each item's merge record (its tile is split), so that the workgroup completing a split tile
  // can fold it; arrival counters start at zero
  {
    std::vector<int32_t> tile_merge(p->tiles.size() / 5, -1);
    p->num_empty_merge = 0;
    for (int32_t k = 0; k < NM; ++k) {
      tile_merge[p->merge_tiles[k]] = k;
      if (p->merge_ptr[k + 1] == p->merge_ptr[k]) ++p->num_empty_merge;
    }
    auto* im = reinterpret_cast<int32_t*>(p->meta.data() + L.imerge);
    for (int32_t k = 0; k < M; ++k) {
      const Item& it = items[p->queue_items[k]];
      im[k] = it.slot >= 0 ? tile_merge[it.tile] : -1;
    }
    p->item_folds = true;
    // the records in LPT order, each with its merge record, so that the decode kernel takes an
    // item with one dependent load
    const auto* lpt = reinterpret_cast<const int32_t*>(p->meta.data() + L.lpt);
    auto* ql = reinterpret_cast<ItemRec*>(p->meta.data() + L.items_lpt);
    for (int32_t t = 0; t < M; ++t) {
      ql[t] = qi[lpt[t]];
      ql[t].pad[0] = im[lpt[t]];
    }
  }
  return BSR_OK;
}

}  // namespace bsr
