// Internal declarations shared by the host planner, the C-ABI layer and the kernels.
// Nothing here is part of the public ABI (include/bsr_attn.h).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "bsr_attn.h"

namespace bsr {

// ---- device metadata records (int32, written by the planner, read by kernels) ----

// Per request: where its queries and pages live.
struct ReqRec {
  int32_t q_start;     // first query row in Q/O
  int32_t q_len;       // l_qo
  int32_t page_start;  // kv_indptr[i]
  int32_t kv_len;      // l_kv
  int32_t tok_start;   // prefix sum of l_kv (debug gather output offset)
  int32_t pad;
  int64_t mask_off;    // first bit of the request's custom mask: sum of l_qo * l_kv before it
};
static_assert(sizeof(ReqRec) == 32, "ReqRec layout");

// Per work item, stored in queue order (worker w runs items [qptr[w], qptr[w+1])).
struct ItemRec {
  int32_t req;
  int32_t row_start;  // packed GQA rows [row_start, row_end) of the request
  int32_t row_end;
  int32_t kv_start;   // logical tokens [kv_start, kv_end) of the request
  int32_t kv_end;
  int32_t slot;       // partial slot, or -1: write the final output
  int32_t q_start;    // the request's first query row, first page-list entry, query and KV
  int32_t page_start; //   lengths, copied from its request record so that the attention kernels
  int32_t q_len;      //   need only this record (the custom-mask offset stays in the request
  int32_t kv_len;     //   record)
  int32_t pad[6];      // (pad[0] of an LPT-ordered copy: the merge record of a split tile, or -1)
};
static_assert(sizeof(ItemRec) == 64, "ItemRec layout");

// Per block of output rows written by the merge pass: a split or empty tile of a plan, or one
// query (all of its GQA rows) of a composable plan.  Slot k of the list holds the partial state of
// rows row_start .. row_end-1 at partial rows (slot * H_kv + h_kv) * T_q + roff_k + (row - row_start),
// with roff_k = 0 unless the record has row offsets (composable plans).
struct MergeRec {
  int32_t q_start;     // first query row in Q/O that packed row 0 refers to
  int32_t row_start;   // packed GQA rows [row_start, row_end): row r is query q_start + r / g,
  int32_t row_end;     //   head g * h_kv + r % g
  int32_t slot_begin;  // into the merge slot list (and the row-offset list)
  int32_t slot_count;  // 0 => empty state
  int32_t has_roff;    // 1: the row-offset list carries roff_k for each slot
  int32_t pad[2];
};
static_assert(sizeof(MergeRec) == 32, "MergeRec layout");

// Ticket counters in a workspace: one pair per group of workgroups that draw from the LPT list.
constexpr int kTicketGroups = 64;

// Byte offsets of the workspace sections (all 256-byte aligned).
struct WsLayout {
  size_t req = 0, indices = 0, items = 0, items_lpt = 0, qptr = 0, merge = 0, mslots = 0, mroff = 0;
  size_t lpt = 0;      // [num_items]: position in `items` of the t-th item in the plan's LPT order
  size_t tickets = 0;  // [kTicketGroups][2]: next ticket, finished workgroups (zero between calls)
  size_t imerge = 0;   // [num_items], queue order: merge record of the item's split tile, or -1
  size_t arrive = 0;   // [num_merge][H_kv]: partial states written so far (zero between calls)
  size_t meta_bytes = 0;  // end of metadata
  size_t part_o = 0, part_lse = 0;
  size_t total = 0;
};

}  // namespace bsr

struct bsr_plan {
  // description
  int32_t B = 0, Hq = 0, Hk = 0, d = 0, P = 1, causal = 0, C = 1, g = 1, Tq = 16;
  int32_t alpha = 2, beta = 1, num_pages = 0;
  int32_t window_left = -1;  // sliding window: keys to the left of the diagonal, -1 = none
  float soft_cap = 0.f;      // logits soft cap, 0 = none
  bool decode = true;  // qo_indptr == NULL
  std::vector<int32_t> qo_indptr, kv_indptr, kv_indices, last_page_len;
  std::vector<int32_t> qo_len, kv_len;
  int64_t mask_bits = 0;  // bits of a custom mask for this plan: sum of l_qo * l_kv
  int32_t max_qo_len = 0;
  int64_t total_kv_tokens = 0;
  // partition
  int64_t W = 0, L = 0;
  std::vector<int32_t> tiles;        // [num_tiles][5]
  std::vector<int32_t> tile_lo;      // [num_tiles]: first visible key of each tile
  std::vector<int32_t> items;        // [num_items][8], creation order
  std::vector<int32_t> queue_ptr;    // [C+1]
  std::vector<int32_t> queue_items;  // [num_items]
  std::vector<int64_t> worker_cost;  // [C]
  std::vector<int32_t> merge_tiles, merge_ptr, merge_slots;
  std::vector<int32_t> merge_roff;   // composable plans: partial-row offset of each merge slot
  int32_t num_slots = 0;
  int32_t num_empty_merge = 0;  // merge records with no slot (tiles with nothing visible)
  bool item_folds = false;      // every split tile's record is reachable from its items (imerge)
  bool affine = false;          // kv_indices was NULL: the identity page table (contiguous KV)
  // composable plans: number of levels and the first (flattened) request of each level
  int32_t num_levels = 1;
  std::vector<int32_t> level_req_start;
  // device image
  bsr::WsLayout ws;
  std::vector<uint8_t> meta;  // host copy of the metadata region (ws.meta_bytes)
  void* pinned = nullptr;     // pinned staging (allocated at first upload)
  void* upload_event = nullptr;
  const void* uploaded_ws = nullptr;
};

namespace bsr {
// host planner (plan.cpp); returns BSR_OK or an error with the message set
int build_plan(const bsr_plan_desc* desc, bsr_plan* p);
// composable plan over several BSR views (compose.cpp)
int build_composable_plan(const bsr_plan_desc* levels, int32_t n_levels, int32_t num_workers, bsr_plan* p);
void set_error(const std::string& msg);
}  // namespace bsr
