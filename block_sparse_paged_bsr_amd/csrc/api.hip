// C ABI of libbsr_attn (include/bsr_attn.h): validation, workspace upload, kernel
// dispatch and optional per-kernel event timing.  No call aborts or throws across the
// ABI; every error returns a bsr_status and leaves a message in bsr_last_error().
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <new>
#include <sstream>
#include <string>
#include <vector>

#include "bsr_internal.h"
#include "kernels/launch.h"

namespace bsr {

static thread_local std::string g_error;
void set_error(const std::string& msg) { g_error = msg; }

namespace {

int hip_fail(const char* what, hipError_t e) {
  std::ostringstream os;
  os << what << ": " << hipGetErrorName(e) << " (" << hipGetErrorString(e) << ")";
  set_error(os.str());
  return BSR_HIP_ERROR;
}

int invalid(const std::string& m) {
  set_error(m);
  return BSR_INVALID_ARG;
}

int unsupported(const std::string& m) {
  set_error(m);
  return BSR_UNSUPPORTED;
}

// ---- optional per-kernel timing ----
struct Timing {
  std::mutex mu;
  bool on = false;
  struct Pair {
    hipEvent_t start, stop;
    int kind;  // 0 attention, 1 merge
  };
  std::vector<Pair> pending;
  double ms[2] = {0.0, 0.0};
  int64_t count[2] = {0, 0};
};
Timing g_timing;

bool timing_on() {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  return g_timing.on;
}

// Records a start event; returns it (or nullptr when timing is off / on failure).
hipEvent_t timing_start(hipStream_t s) {
  if (!timing_on()) return nullptr;
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  if (hipEventRecord(e, s) != hipSuccess) {
    (void)hipEventDestroy(e);
    return nullptr;
  }
  return e;
}

void timing_stop(hipEvent_t start, hipStream_t s, int kind) {
  if (!start) return;
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess || hipEventRecord(e, s) != hipSuccess) {
    if (e) (void)hipEventDestroy(e);
    (void)hipEventDestroy(start);
    return;
  }
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.pending.push_back({start, e, kind});
}

int p_shift_of(int P) {
  if (P <= 0 || (P & (P - 1))) return -1;
  int s = 0;
  while ((1 << s) < P) ++s;
  return s;
}

RunArgs make_args(const bsr_plan* p, const void* ws) {
  const char* base = static_cast<const char*>(ws);
  RunArgs a{};
  a.req = reinterpret_cast<const ReqRec*>(base + p->ws.req);
  a.indices = reinterpret_cast<const int32_t*>(base + p->ws.indices);
  a.items = reinterpret_cast<const ItemRec*>(base + p->ws.items);
  a.qptr = reinterpret_cast<const int32_t*>(base + p->ws.qptr);
  a.merge = reinterpret_cast<const MergeRec*>(base + p->ws.merge);
  a.mslots = reinterpret_cast<const int32_t*>(base + p->ws.mslots);
  a.mroff = reinterpret_cast<const int32_t*>(base + p->ws.mroff);
  a.lpt = reinterpret_cast<const int32_t*>(base + p->ws.lpt);
  a.items_lpt = reinterpret_cast<const ItemRec*>(base + p->ws.items_lpt);
  a.tickets = reinterpret_cast<int32_t*>(const_cast<char*>(base) + p->ws.tickets);
  a.num_items = int32_t(p->items.size() / 8);
  a.imerge = reinterpret_cast<const int32_t*>(base + p->ws.imerge);
  a.arrive = reinterpret_cast<int32_t*>(const_cast<char*>(base) + p->ws.arrive);
  a.fold_in_kernel = 0;
  a.affine = p->affine ? 1 : 0;
  a.part_o = reinterpret_cast<float*>(const_cast<char*>(base) + p->ws.part_o);
  a.part_lse = reinterpret_cast<float*>(const_cast<char*>(base) + p->ws.part_lse);
  a.B = p->B;
  a.Hq = p->Hq;
  a.Hk = p->Hk;
  a.g = p->g;
  a.d = p->d;
  a.P = p->P;
  a.Tq = p->Tq;
  a.C = p->C;
  a.causal = p->causal;
  a.num_merge = int32_t(p->merge_tiles.size());
  a.p_shift = p_shift_of(p->P);
  a.window_left = p->window_left;
  a.soft_cap = p->soft_cap;
  a.k_scale = 1.f;
  a.v_scale = 1.f;
  return a;
}

bool positive_finite(float x) { return x > 0.f && x != __builtin_huge_valf(); }

// kv_e4m3: K and V are E4M3 bytes with per-tensor scales (decode only; Q and O are bf16).
// ws_ready: the caller has just copied the plan's metadata into ws (the static-scratch entry).
int run_common(const bsr_plan* p, const void* ws, const void* q, const void* k, const void* v,
               void* o, float* lse, int32_t dtype, float sm_scale, void* stream, bool decode_call,
               bool kv_e4m3 = false, float k_scale = 1.f, float v_scale = 1.f,
               const uint8_t* mask = nullptr, bool ws_ready = false) {
  if (!p) return invalid("plan is NULL");
  if (!ws) return invalid("workspace is NULL");
  if (!ws_ready && ws != p->uploaded_ws)
    return invalid("workspace was not uploaded for this plan (call bsr_plan_upload first)");
  if (dtype != BSR_DTYPE_F32 && dtype != BSR_DTYPE_BF16) return invalid("unknown dtype");
  if (decode_call && !p->decode)
    return invalid("bsr_run_decode needs a plan with one query per request (qo_indptr == NULL); use bsr_run_prefill");
  if (!positive_finite(sm_scale)) return invalid("sm_scale must be positive and finite");
  if (kv_e4m3 && !(positive_finite(k_scale) && positive_finite(v_scale)))
    return invalid("k_scale and v_scale must be positive and finite");
  if (kv_e4m3 && !decode_bf16_supported(p->d, p->g, p->Tq))
    return unsupported("e4m3 KV decode needs head_dim 64 or 128 and at most 16 query heads per KV head "
                       "(and a query tile of at least that many rows)");
  if (p->B == 0) return BSR_OK;
  if (!q || !k || !v || !o || !lse) return invalid("q, k_cache, v_cache, o and lse must be non-NULL");
  const bool any_tokens = p->total_kv_tokens > 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  RunArgs a = make_args(p, ws);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.sm_scale = sm_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.mask = mask;

  hipError_t e = hipSuccess;
  if (!p->items.empty()) {
    hipEvent_t t0 = timing_start(s);
    // split tiles of a plan on the decode kernel (bf16 or E4M3 KV) are folded by the wave that
    // writes a tile's last partial state (partial states addressed with 32-bit offsets)
    const bool fold_ok = p->item_folds && size_t(p->Hk) * p->Tq * (p->d + 1) * sizeof(float) * p->num_slots < (size_t(1) << 31);
    if (kv_e4m3) {
      a.fold_in_kernel = fold_ok ? 1 : 0;
      e = launch_decode_bf16(a, true, s);
    } else if (dtype == BSR_DTYPE_F32) {
      if (!attn_f32_supported(p->d)) return unsupported("fp32 head_dim must be one of 16, 32, 64, 128, 256");
      e = launch_attn_f32(a, s);
    } else {
      // the decode kernel (no custom-mask, causal or window path) serves decode plans and
      // non-causal plans of tiles of at most 16 packed rows; everything else the tiled kernels
      const bool dec_ok = !mask && ((p->decode && decode_bf16_supported(p->d, p->g, p->Tq)) ||
                                    (!p->causal && p->window_left < 0 && decode_bf16_tiles(p->d, p->g, p->Tq)));
      if (dec_ok) {
        a.fold_in_kernel = fold_ok ? 1 : 0;
        e = launch_decode_bf16(a, false, s);
      } else {
        if (!prefill_bf16_supported(p->d, p->Tq)) return unsupported("bf16 head_dim must be 64 or 128");
        e = launch_prefill_bf16(a, s);
      }
    }
    timing_stop(t0, s, 0);
    if (e != hipSuccess) return hip_fail("attention kernel launch", e);
  } else if (dtype == BSR_DTYPE_BF16 && !prefill_bf16_supported(p->d, p->Tq)) {
    return unsupported("bf16 head_dim must be 64 or 128");
  } else if (dtype == BSR_DTYPE_F32 && !attn_f32_supported(p->d)) {
    return unsupported("fp32 head_dim must be one of 16, 32, 64, 128, 256");
  }
  (void)any_tokens;
  const int32_t merge_left = a.fold_in_kernel ? p->num_empty_merge : a.num_merge;  // records for the merge pass
  if (merge_left > 0) {
    hipEvent_t t1 = timing_start(s);
    e = launch_merge(a, dtype, s);
    timing_stop(t1, s, 1);
    if (e != hipSuccess) return hip_fail("merge kernel launch", e);
  }
  return BSR_OK;
}

// ---- the static scratch of bsr_run_decode_scratch ----
// For callers that cannot allocate device memory: a file-scope device array that every GPU the
// library runs on holds from module load until the process ends.  Host code never passes its
// name to a kernel or a copy: the array's device address on the current GPU comes from
// hipGetSymbolAddress, once per device, and is kept in g_scratch.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) return unsupported("device index beyond the library's scratch table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return BSR_OK;
}

}  // namespace
}  // namespace bsr

using namespace bsr;

extern "C" {

const char* bsr_last_error(void) { return g_error.c_str(); }

const char* bsr_version(void) { return "bsr_attn 0.1.0 (gfx950)"; }

int bsr_plan_create(const bsr_plan_desc* desc, bsr_plan** out) {
  if (!out) return invalid("out is NULL");
  *out = nullptr;
  bsr_plan* p = new (std::nothrow) bsr_plan();
  if (!p) return invalid("out of host memory");
  int rc;
  try {
    rc = build_plan(desc, p);
  } catch (const std::bad_alloc&) {
    set_error("out of host memory while planning");
    rc = BSR_INVALID_ARG;
  }
  if (rc != BSR_OK) {
    delete p;
    return rc;
  }
  *out = p;
  return BSR_OK;
}

int bsr_plan_create_composable(const bsr_plan_desc* levels, int32_t n_levels, int32_t num_workers, bsr_plan** out) {
  if (!out) return invalid("out is NULL");
  *out = nullptr;
  bsr_plan* p = new (std::nothrow) bsr_plan();
  if (!p) return invalid("out of host memory");
  int rc;
  try {
    rc = build_composable_plan(levels, n_levels, num_workers, p);
  } catch (const std::bad_alloc&) {
    set_error("out of host memory while planning");
    rc = BSR_INVALID_ARG;
  }
  if (rc != BSR_OK) {
    delete p;
    return rc;
  }
  *out = p;
  return BSR_OK;
}

void bsr_plan_destroy(bsr_plan* p) {
  if (!p) return;
  if (p->upload_event) {
    (void)hipEventSynchronize(static_cast<hipEvent_t>(p->upload_event));
    (void)hipEventDestroy(static_cast<hipEvent_t>(p->upload_event));
  }
  if (p->pinned) (void)hipHostFree(p->pinned);
  delete p;
}

int bsr_plan_workspace_bytes(const bsr_plan* p, size_t* bytes) {
  if (!p || !bytes) return invalid("plan and bytes must be non-NULL");
  *bytes = p->ws.total;
  return BSR_OK;
}

int bsr_plan_upload(bsr_plan* p, void* dev_ws, size_t ws_bytes, void* stream) {
  if (!p || !dev_ws) return invalid("plan and dev_ws must be non-NULL");
  if (ws_bytes < p->ws.total) {
    std::ostringstream os;
    os << "workspace has " << ws_bytes << " bytes, the plan needs " << p->ws.total;
    set_error(os.str());
    return BSR_CAPACITY;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (!p->pinned) {
    e = hipHostMalloc(&p->pinned, p->meta.size(), hipHostMallocDefault);
    if (e != hipSuccess) {
      p->pinned = nullptr;
      return hip_fail("hipHostMalloc(plan staging)", e);
    }
    std::memcpy(p->pinned, p->meta.data(), p->meta.size());
  }
  if (!p->upload_event) {
    hipEvent_t ev;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail("hipEventCreate", e);
    p->upload_event = ev;
  }
  e = hipMemcpyAsync(dev_ws, p->pinned, p->meta.size(), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail("hipMemcpyAsync(plan upload)", e);
  e = hipEventRecord(static_cast<hipEvent_t>(p->upload_event), s);
  if (e != hipSuccess) return hip_fail("hipEventRecord", e);
  p->uploaded_ws = dev_ws;
  return BSR_OK;
}

int bsr_plan_export(const bsr_plan* p, bsr_plan_view* v) {
  if (!p || !v) return invalid("plan and view must be non-NULL");
  v->batch = p->B;
  v->num_qo_heads = p->Hq;
  v->num_kv_heads = p->Hk;
  v->head_dim = p->d;
  v->page_size = p->P;
  v->causal = p->causal;
  v->group_size = p->g;
  v->tile_q = p->Tq;
  v->num_workers = p->C;
  v->num_slots = p->num_slots;
  v->total_work = p->W;
  v->chunk_limit = p->L;
  v->num_tiles = int32_t(p->tiles.size() / 5);
  v->tiles = p->tiles.data();
  v->num_items = int32_t(p->items.size() / 8);
  v->items = p->items.data();
  v->queue_ptr = p->queue_ptr.data();
  v->queue_items = p->queue_items.data();
  v->worker_cost = p->worker_cost.data();
  v->num_merge = int32_t(p->merge_tiles.size());
  v->merge_tiles = p->merge_tiles.data();
  v->merge_ptr = p->merge_ptr.data();
  v->merge_slots = p->merge_slots.data();
  v->window_left = p->window_left;
  v->logits_soft_cap = p->soft_cap;
  v->tile_lo = p->tile_lo.data();
  v->custom_mask_bits = p->mask_bits;
  v->num_levels = p->num_levels;
  v->level_req_start = p->level_req_start.empty() ? nullptr : p->level_req_start.data();
  v->merge_row_off = p->merge_roff.empty() ? nullptr : p->merge_roff.data();
  return BSR_OK;
}

int bsr_run_decode(const bsr_plan* plan, const void* ws, const void* q, const void* k_cache,
                   const void* v_cache, void* o, float* lse, int32_t dtype, float sm_scale,
                   void* stream) {
  return run_common(plan, ws, q, k_cache, v_cache, o, lse, dtype, sm_scale, stream, true);
}

int bsr_run_decode_scratch(const bsr_plan* plan, const void* q, const void* k_cache, const void* v_cache,
                           void* o, float* lse, int32_t dtype, float sm_scale, void* stream) {
  if (!plan) return invalid("plan is NULL");
  if (plan->ws.total > kScratchBytes) {
    std::ostringstream os;
    os << "the plan needs " << plan->ws.total << " bytes of workspace; bsr_run_decode_scratch holds at most "
       << kScratchBytes << " (use bsr_run_decode with a workspace of that size)";
    set_error(os.str());
    return BSR_CAPACITY;
  }
  if (!plan->decode)
    return invalid("bsr_run_decode_scratch needs a plan with one query per request (qo_indptr == NULL)");
  if (plan->B == 0) return BSR_OK;
  void* ws = nullptr;
  int rc = scratch_on_current_device(&ws);
  if (rc != BSR_OK) return rc;
  // this call's plan metadata into the scratch (stream-ordered; partial states need no clearing:
  // the merge reads only slots the attention kernel wrote in the same call)
  const void* src = plan->pinned ? plan->pinned : static_cast<const void*>(plan->meta.data());
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(ws, src, plan->meta.size(), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail("hipMemcpyAsync(plan metadata into the scratch)", e);
  return run_common(plan, ws, q, k_cache, v_cache, o, lse, dtype, sm_scale, stream, true, false, 1.f, 1.f,
                    nullptr, true);
}

int bsr_run_prefill_masked(const bsr_plan* plan, const void* ws, const void* q, const void* k_cache,
                           const void* v_cache, const void* mask, void* o, float* lse, int32_t dtype,
                           float sm_scale, void* stream) {
  if (plan && plan->mask_bits > 0 && !mask) return invalid("mask is NULL");
  return run_common(plan, ws, q, k_cache, v_cache, o, lse, dtype, sm_scale, stream, false, false, 1.f, 1.f,
                    static_cast<const uint8_t*>(mask));
}

int bsr_run_decode_e4m3(const bsr_plan* plan, const void* ws, const void* q, const void* k_cache,
                        const void* v_cache, void* o, float* lse, float sm_scale, float k_scale,
                        float v_scale, void* stream) {
  return run_common(plan, ws, q, k_cache, v_cache, o, lse, BSR_DTYPE_BF16, sm_scale, stream, true, true,
                    k_scale, v_scale);
}

int bsr_run_prefill(const bsr_plan* plan, const void* ws, const void* q, const void* k_cache,
                    const void* v_cache, void* o, float* lse, int32_t dtype, float sm_scale,
                    void* stream) {
  return run_common(plan, ws, q, k_cache, v_cache, o, lse, dtype, sm_scale, stream, false);
}

int bsr_merge_state(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    void* o_out, float* lse_out, int64_t rows, int32_t heads, int32_t head_dim,
                    int32_t dtype, void* stream) {
  if (rows < 0 || heads < 0 || head_dim < 1) return invalid("rows, heads must be >= 0 and head_dim >= 1");
  if (dtype != BSR_DTYPE_F32 && dtype != BSR_DTYPE_BF16) return invalid("unknown dtype");
  if (rows * int64_t(heads) > (int64_t(1) << 31) / 16) return invalid("too many states");
  if (rows * heads == 0) return BSR_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return invalid("NULL state pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_merge_state(o_a, lse_a, o_b, lse_b, o_out, lse_out, rows, heads, head_dim, dtype, s);
  if (e != hipSuccess) return hip_fail("merge_state launch", e);
  return BSR_OK;
}

int bsr_debug_gather_rows(const bsr_plan* p, const void* ws, int64_t* rows_dev, void* stream) {
  if (!p || !ws) return invalid("plan and ws must be non-NULL");
  if (ws != p->uploaded_ws) return invalid("workspace was not uploaded for this plan");
  if (p->total_kv_tokens == 0) return BSR_OK;
  if (!rows_dev) return invalid("rows_dev is NULL");
  RunArgs a = make_args(p, ws);
  hipError_t e = launch_gather_rows(a, rows_dev, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail("gather_rows launch", e);
  return BSR_OK;
}

int bsr_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (auto& pr : g_timing.pending) {
    (void)hipEventDestroy(pr.start);
    (void)hipEventDestroy(pr.stop);
  }
  g_timing.pending.clear();
  g_timing.ms[0] = g_timing.ms[1] = 0.0;
  g_timing.count[0] = g_timing.count[1] = 0;
  g_timing.on = on != 0;
  return BSR_OK;
}

int bsr_timing_read(double* attn_ms, int64_t* attn_launches, double* merge_ms, int64_t* merge_launches) {
  std::lock_guard<std::mutex> lk(g_timing.mu);
  for (auto& pr : g_timing.pending) {
    hipError_t e = hipEventSynchronize(pr.stop);
    if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, pr.start, pr.stop);
    if (e != hipSuccess) return hip_fail("hipEventElapsedTime", e);
    g_timing.ms[pr.kind] += ms;
    g_timing.count[pr.kind] += 1;
    (void)hipEventDestroy(pr.start);
    (void)hipEventDestroy(pr.stop);
  }
  g_timing.pending.clear();
  if (attn_ms) *attn_ms = g_timing.ms[0];
  if (attn_launches) *attn_launches = g_timing.count[0];
  if (merge_ms) *merge_ms = g_timing.ms[1];
  if (merge_launches) *merge_launches = g_timing.count[1];
  return BSR_OK;
}

int bsr_query_num_workers(int32_t device, int32_t kind, int32_t num_qo_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t* out) {
  if (!out || num_kv_heads < 1 || num_qo_heads < 1 || num_qo_heads % num_kv_heads)
    return invalid("bad arguments to bsr_query_num_workers");
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_fail("hipDeviceGetAttribute", e);
  const int g = num_qo_heads / num_kv_heads;
  int per_cu = 1, per_worker = num_kv_heads;
  if (kind == 0 && decode_bf16_supported(head_dim, g, 128)) {
    per_cu = decode_bf16_blocks_per_cu(head_dim, num_kv_heads);
    per_worker = decode_bf16_blocks_per_worker(num_kv_heads);
  } else if (head_dim == 64 || head_dim == 128) {
    per_cu = prefill_bf16_blocks_per_cu(head_dim);
  }
  *out = std::max(1, cus * per_cu / per_worker);
  return BSR_OK;
}

}  // extern "C"
