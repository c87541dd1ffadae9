// bf16 paged decode on gfx950: one query token per request, GQA-fused, split-KV.
//
// Decode reads every KV byte once and does O(g) arithmetic per byte (operational
// intensity O(g * l_qo): "FlashInfer: Engineering a Customizable, Block-Sparse
// Attention Engine for LLM Inference Serving" §II.3-II.4; eq. 2 of "FlashInfer:
// Making Attention Fit the Serving Workload"), so the kernel is organised around HBM
// traffic: one wave streams the KV rows of one KV head once and serves all g <= 16
// query heads of the group with them (head-group fusion, eq. 3 of the review).
//
// A 16-token step, lane = n + 16 j (n = 0..15, j = 0..3):
//   loads   K[token n][kb*32 + j*8 .. +8] and V[token n][kb*32 + j*8 .. +8] for
//           kb = 0 .. D/32-1, 16 bytes each, rows found through the page table (eq. 7);
//           the next step's rows are requested before the current step is computed.
//   scores  S^T = K Q^T on v_mfma_f32_16x16x32_bf16: the K fragment is the A operand
//           as loaded, Q^T (column n = packed row n of the tile: one of the g query heads, or
//           of the rows of a several-query tile) is the B operand; lane (n, j) receives the
//           scores of tokens 4j..4j+3 for row n.
//   softmax per head (one column per lane group), in log2 units, with the running
//           maximum of the online-softmax recurrence ("FlashInfer: Engineering ...",
//           §II.2); the accumulator is rescaled only when the maximum grows.
//   output  O^T += V^T P^T on v_mfma_f32_16x16x16_bf16: P^T is the score accumulator
//           converted to bf16 in place (B operand), V^T comes from the step's V rows
//           staged in a wave-private LDS tile and read back with the transposing
//           LDS read of gfx950 (ds_read_b64_tr_b16, A operand).
// A work item writes the final (O, LSE) or a partial state.  The partial states of a split tile
// are folded by the workgroup that writes the tile's last one (see fold_tile below); the merge
// pass then only writes tiles with nothing visible.
// CAP: logits soft cap (eq. 8 of the review), each scaled score s becomes c tanh(s / c).  A
// sliding window needs nothing here: all rows of a decode item share one query position, so
// the planned chunks already start at the window.
// KV8: K and V stored as E4M3 bytes (OCP "FN" encoding) with one scale per tensor, the e4m3
// KV cache of the review's vLLM integration (Appendix G.4).  A lane's 16-byte load then holds
// 16 values of a row (two k-blocks of the score product; Q is loaded in the same order), and
// v_cvt_scalef32_pk_bf16_fp8 (scale 1) widens each pair exactly to the bf16 operands.  The K
// scale is folded into the score scale and the V scale into the output normalisation, so the
// loop does no extra multiplications; the bytes read per token are half of bf16's, and a step
// covers 32 tokens (two 16-token halves loaded together) to keep a bf16 step's bytes in flight.
#include <algorithm>
#include <climits>

#include "common.h"
#include "launch.h"

namespace bsr {

// four E4M3 bytes -> four bf16 values (exact: every E4M3 value is a bf16 value), as two packed
// pairs, by gfx950's scaled pair conversion with a scale of 1
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true))};
}

// A workgroup serves up to kDecodeWaves KV heads of one worker, one wave per head: its waves run
// the same work items over the same tokens, so together they read whole token rows (all KV heads
// of a token are adjacent, 2 KB at 8 heads x 128 bf16) and whole pages at about the same time,
// instead of one head's 256-byte slice of each row from a workgroup of its own.
constexpr int kDecodeWaves = 8;

template <int D>
constexpr int decode_vs_bytes() { return 16 * (D + 8) * 2; }  // one wave's V staging tile

// Buffer resources over the partial states (raw, byte offsets; the host keeps them below 2 GiB)
// and the cache policy of their accesses: agent scope (sc1), the encoding the compiler gives a
// relaxed agent-scope atomic load or store, so that every access is coherent across the XCDs'
// separate L2 caches without a whole-cache write-back or invalidation.
constexpr int kAgentScope = 16;  // sc1
// partial states whose loads a folding lane issues together
constexpr int kFoldSlots = 8;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, 0x7fffffff, 0x00020000);
}
#define BSR_DECODE_WAIT_VMCNT0() __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8))
// vmcnt(n) for n < 16 (lgkmcnt and expcnt not waited for)
#define BSR_DECODE_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8) | ((n) & 15))

// FOLD: the plan's split tiles are folded inside this kernel (RunArgs::fold_in_kernel); without
// it the kernel carries no fold code, and the merge pass folds them.  AFF: the cache is
// contiguous (RunArgs::affine), so page ids are computed instead of loaded from the table.
template <int D, bool CAP, bool KV8, bool FOLD, bool AFF>
__global__ __launch_bounds__(64 * kDecodeWaves) void attn_decode_bf16_kernel(RunArgs a) {
  constexpr int KB = D / 32;  // k-blocks of the score product
  constexpr int DB = D / 16;  // d-blocks of the output product
  constexpr int VS = D + 8;   // LDS row stride (elements); 16-byte aligned rows
  constexpr int ES = KV8 ? 1 : 2;                // bytes per K/V element
  constexpr int NL = KV8 ? D / 64 : D / 32;      // 16-byte loads per row and lane (64 j-apart bytes)
  constexpr int PD = KV8 ? 2 : 1;  // 16-token halves per step (E4M3 rows are half as long)
  extern __shared__ __attribute__((aligned(16))) uint16_t decode_lds[];

  __shared__ int s_ticket;
  const int wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const int hk = blockIdx.y * waves + wave;  // (waves divides H_kv: every wave has a head)
  // the wave's private V tile; LDS operations of one wave complete in order, so staging and the
  // transposing reads need no barrier
  uint16_t* Vs = decode_lds + wave * (16 * VS);
  const int lane = threadIdx.x & 63, n = lane & 15, j = lane >> 4;
  const int g = a.g;
  const float qk_scale = KV8 ? a.sm_scale * a.k_scale : a.sm_scale;  // K's scale joins the score scale
  const float c = CAP ? qk_scale / a.soft_cap : qk_scale * kLog2e;
  const float cap_l2 = a.soft_cap * kLog2e;
  const float o_scale = KV8 ? a.v_scale : 1.f;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint8_t* __restrict__ K = static_cast<const uint8_t*>(a.k);
  const uint8_t* __restrict__ V = static_cast<const uint8_t*>(a.v);
  uint16_t* __restrict__ O = static_cast<uint16_t*>(a.o);
  const __amdgpu_buffer_rsrc_t part_o_rs = raw_rsrc(a.part_o), part_lse_rs = raw_rsrc(a.part_lse);

  // Column n of an item serves packed row row_start + n of its tile (GQA packing, eq. 3 of the
  // review): query q_start + row / g, head g * h_kv + row % g.  A decode tile is the g heads of one
  // query; a tile of a non-causal block row of several queries (the shared level of a composable
  // format) holds up to 16 rows.  Columns past the tile repeat one of its rows.
  auto out_row = [&](const ItemRec& itm) -> int64_t {
    const int rows = itm.row_end - itm.row_start;
    const int row = itm.row_start + (n < rows ? n : n % rows);
    return int64_t(itm.q_start + row / g) * a.Hq + hk * g + row % g;
  };
  // Q^T as the B operand: column n = that row's query and head; k-block kb covers the head-dim
  // values this lane's K slice of that block holds
  auto load_q = [&](const ItemRec& itm, bf16x8 (&dst)[KB]) {
    const uint16_t* qp = Q + out_row(itm) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int col = KV8 ? 64 * (kb >> 1) + 16 * j + 8 * (kb & 1) : 32 * kb + 8 * j;
      dst[kb] = *reinterpret_cast<const bf16x8*>(qp + col);
    }
  };
  // page of token t of an item (eq. 7), t clamped to the item's last token; a contiguous cache
  // (identity page table) computes it without the table's load, the affine addressing of
  // "FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for LLM Inference
  // Serving" §V.4
  auto page_in = [&](const ItemRec& itm, int t) -> int32_t {
    const int tc = min(t, itm.kv_end - 1);
    const int32_t x = itm.page_start + (a.p_shift >= 0 ? (tc >> a.p_shift) : tc / a.P);
    return AFF ? x : a.indices[x];
  };

  // Work distribution: the plan's items in its LPT order (longest first), taken by whichever
  // workgroup is free through a ticket counter -- the order of the longest-processing-time
  // partition, without binding an item to a worker in advance, so that compute units running at
  // different clocks finish together.  Every item writes its own output or partial slot and the
  // merge folds slots in the plan's order, so the results do not depend on which workgroup ran
  // which item.  All waves of a workgroup (one per KV head) take the same item.  The last
  // workgroup to find the list exhausted returns the counters to zero for the next call.
  // The work item record carries everything this kernel needs (rows, KV range, slot, query and
  // page-list starts).  The next item is claimed and its record fetched in the second-to-last step
  // of the current one, and its queries and first page ids issued in the last step, so that a new
  // item starts with only its first rows to wait for.  The grid's workgroups are all resident and
  // start together, so the first round needs no counter: workgroup b takes ticket b, and the
  // counter hands out tickets gridDim.x, gridDim.x + 1, ... to the workgroups that finish first
  // (no burst of atomics on one address at the start of every call).
  int32_t* tk = a.tickets + 2 * blockIdx.y;
  auto draw = [&]() -> int {
    if (threadIdx.x == 0)
      s_ticket = int(gridDim.x) + __hip_atomic_fetch_add(tk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int t = s_ticket;
    __syncthreads();  // every wave has read it before the next draw writes it
    return t;
  };
  constexpr int NPRE = KV8 ? 4 : 2;  // page ids of the first two steps (16 tokens each)
  const int num_items = a.num_items;
  int t = blockIdx.x;
  ItemRec next = a.items_lpt[t < num_items ? t : 0];
  int next_mi = FOLD ? next.pad[0] : -1;
  bf16x8 qb[KB], qn[KB];
  int32_t pre[NPRE];
  bool have_pre = false;
  // the next item's first rows (E4M3: its first two 16-token halves) when a folding item issued
  // them before its count
  u32x4 kr0[PD][NL], vr0[PD][NL];
  bool have_rows = false;
  while (t < num_items) {
    const ItemRec item = next;
    const int item_mi = next_mi;
    bool claimed = false, more = false;
    auto claim = [&]() {  // every wave of the workgroup reaches this at the same step of the item
      t = draw();
      more = t < num_items;
      if (more) {
        next = a.items_lpt[t];
        if constexpr (FOLD) next_mi = next.pad[0];
      }
      claimed = true;
    };
    const int kv_end = item.kv_end;
    const int64_t orow = out_row(item);
    // a split tile's merge record and its first slot ids (lane u < kFoldSlots: slot id u), read
    // at the item's start so that no load has to complete between the item's last stores and
    // its count
    int fold_ns = 0, fold_begin = 0, fold_sid = 0;
    if constexpr (FOLD) {
      if (item_mi >= 0) {
        const MergeRec mr = a.merge[item_mi];
        fold_ns = mr.slot_count;
        fold_begin = mr.slot_begin;
        fold_sid = a.mslots[fold_begin + min(lane % kFoldSlots, fold_ns - 1)];
      }
    }
    if (have_pre) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) qb[kb] = qn[kb];
    } else {
      load_q(item, qb);
#pragma unroll
      for (int u = 0; u < NPRE; ++u) pre[u] = page_in(item, item.kv_start + 16 * u + n);
    }
    have_pre = false;
    // the next item's queries and first page ids (issued in this item's last step)
    auto preload_next = [&]() {
      if (!more) return;
      load_q(next, qn);
#pragma unroll
      for (int u = 0; u < NPRE; ++u) pre[u] = page_in(next, next.kv_start + 16 * u + n);
      have_pre = true;
    };

    float m = kNegInf, l = 0.f;
    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    // page of this lane's token (lane n of a step): the index load runs one step ahead of
    // the row loads, which run one step ahead of the computation
    auto page_of = [&](int t) -> int32_t { return page_in(item, t); };
    // byte offset of this lane's first 16-byte piece of token t's row
    auto row_base = [&](int t, int32_t page, int kend) -> int64_t {
      const int tc = min(t, kend - 1);
      const int off = a.p_shift >= 0 ? (tc & ((1 << a.p_shift) - 1)) : tc - (tc / a.P) * a.P;
      return ((int64_t(page) * a.P + off) * a.Hk + hk) * (D * ES) + j * 16;
    };
    // bf16 V rows go through LDS anyway, so their loads read whole pieces of the token slices:
    // load i of a step reads tokens TPI i .. TPI i + TPI - 1 of the step, lane (vt, vc) the
    // 16-byte chunk vc of token TPI i + vt (one instruction covers whole 128-byte lines), with
    // that token's page taken from the lane that looked it up
    constexpr int CPT = D / 8, TPI = 64 / CPT;  // 16-byte chunks per slice, tokens per load
    static_assert(KV8 || TPI * NL == 16, "one step's 16 tokens in NL loads");
    static_assert(2 * NL * PD < 16, "the rows of one step fit the vmcnt field of the fold's wait");
    const int vt = lane / CPT, vc = lane % CPT;
    auto load_rows = [&](u32x4 (&kd)[NL], u32x4 (&vd)[NL], int t, int32_t page, int kend) {
      const int64_t base = row_base(t, page, kend);
#pragma unroll
      for (int l = 0; l < NL; ++l) kd[l] = *reinterpret_cast<const u32x4*>(K + base + 64 * l);
      if constexpr (KV8) {
#pragma unroll
        for (int l = 0; l < NL; ++l) vd[l] = *reinterpret_cast<const u32x4*>(V + base + 64 * l);
      } else {
        const int ts = t - n;  // the step's first token (lane n carries token ts + n)
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int tok = TPI * i + vt;
          const int32_t pg = __shfl(page, tok, 64);
          vd[i] = *reinterpret_cast<const u32x4*>(V + row_base(ts + tok, pg, kend) - j * 16 + vc * 16);
        }
      }
    };
    // one step: tokens t0 .. t0 + 15 (lane n: token t0 + n) from the rows in kr / vr
    auto compute = [&](int t0, const u32x4 (&kr)[NL], const u32x4 (&vr)[NL]) {
      // scores S^T[token 4j+i][head n]
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        u32x4 ka;
        if constexpr (KV8) {
          const u32x4 w = kr[kb >> 1];
          const u32x2 x0 = e4m3x4_to_bf16x4(w[2 * (kb & 1)]), x1 = e4m3x4_to_bf16x4(w[2 * (kb & 1) + 1]);
          ka = u32x4{x0[0], x0[1], x1[0], x1[1]};
        } else {
          ka = kr[kb];
        }
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka), qb[kb], S, 0, 0, 0);
      }

      // stage V rows (token n) as bf16 for the transposing read below (the previous step's
      // reads of the tile were issued before these writes and complete first)
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        if constexpr (KV8) {
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const u32x2 x0 = e4m3x4_to_bf16x4(vr[l][2 * hb]), x1 = e4m3x4_to_bf16x4(vr[l][2 * hb + 1]);
            *reinterpret_cast<u32x4*>(Vs + n * VS + 64 * l + 16 * j + 8 * hb) = u32x4{x0[0], x0[1], x1[0], x1[1]};
          }
        } else {
          *reinterpret_cast<u32x4*>(Vs + (TPI * l + vt) * VS + 8 * vc) = vr[l];
        }
      }

      float s[4];
      float mt = kNegInf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float si = CAP ? cap_l2 * fast_tanh(S[i] * c) : S[i] * c;
        s[i] = (t0 + 4 * j + i) < kv_end ? si : kNegInf;
        mt = fmaxf(mt, s[i]);
      }
      mt = fmaxf(mt, shfl_xor(mt, 16));
      mt = fmaxf(mt, shfl_xor(mt, 32));
      if (mt > m) {  // the running maximum grew: rescale this head's state
        const float corr = exp2f(m - mt);
        l *= corr;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= corr;
        m = mt;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = exp2f(s[i] - m);
        l += p[i];
      }
      const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])});
      // V^T operand: ds_read_b64_tr_b16 gives lane 16G+i the values V[token 4G+e][d0+i],
      // e = 0..3, when lane 16G+4e+q addresses V[token 4G+e][d0+4q .. +4]
      const uint16_t* vtr = Vs + (4 * j + ((lane >> 2) & 3)) * VS + 4 * (lane & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vtr + db * 16));
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[db], 0, 0, 0);
      }
    };

    if constexpr (PD == 1) {
      int32_t pg_next = pre[1];
      u32x4 kr[NL], vr[NL];
      if (have_rows) {
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          kr[l] = kr0[0][l];
          vr[l] = vr0[0][l];
        }
      } else {
        load_rows(kr, vr, item.kv_start + n, pre[0], kv_end);
      }
      have_rows = false;
      for (int t0 = item.kv_start; t0 < kv_end; t0 += 16) {
        const bool has_next = t0 + 16 < kv_end;
        const int32_t pg_after = page_of(t0 + 32 + n);
        // request the next step's rows (or, in the last step, the next item's queries and first
        // page ids) before touching this step's data
        u32x4 kn[NL], vn[NL];
        if (has_next) load_rows(kn, vn, t0 + 16 + n, pg_next, kv_end);
        if (!claimed && t0 + 32 >= kv_end) claim();
        if (!has_next) preload_next();
        pg_next = pg_after;
        compute(t0, kr, vr);
        if (has_next) {
#pragma unroll
          for (int l = 0; l < NL; ++l) {
            kr[l] = kn[l];
            vr[l] = vn[l];
          }
        }
      }
    } else {
      // E4M3: 32 tokens per step, two 16-token halves loaded together, so a wave has as many
      // bytes in flight as with one step of bf16 rows
      int32_t pg_next0 = pre[2], pg_next1 = pre[3];
      u32x4 kr[2][NL], vr[2][NL];
      if (have_rows) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int l = 0; l < NL; ++l) {
            kr[h2][l] = kr0[h2][l];
            vr[h2][l] = vr0[h2][l];
          }
      } else {
        load_rows(kr[0], vr[0], item.kv_start + n, pre[0], kv_end);
        load_rows(kr[1], vr[1], item.kv_start + 16 + n, pre[1], kv_end);
      }
      have_rows = false;
      for (int t0 = item.kv_start; t0 < kv_end; t0 += 32) {
        const bool has_next = t0 + 32 < kv_end;
        const int32_t pa0 = page_of(t0 + 64 + n), pa1 = page_of(t0 + 80 + n);
        // (unconditional: past the end the rows clamp to the chunk's last row)
        u32x4 kn[2][NL], vn[2][NL];
        load_rows(kn[0], vn[0], t0 + 32 + n, pg_next0, kv_end);
        load_rows(kn[1], vn[1], t0 + 48 + n, pg_next1, kv_end);
        if (!claimed && t0 + 64 >= kv_end) claim();
        if (!has_next) preload_next();
        compute(t0, kr[0], vr[0]);
        if (t0 + 16 < kv_end) compute(t0 + 16, kr[1], vr[1]);
        pg_next0 = pa0;
        pg_next1 = pa1;
        (void)has_next;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int l = 0; l < NL; ++l) {
            kr[h2][l] = kn[h2][l];
            vr[h2][l] = vn[h2][l];
          }
      }
    }

    if (!claimed) claim();  // (an item always reaches its last step; kept for safety)
    // lane (n, j) summed tokens 4j..4j+3 of every step; add the four token groups
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    // a split item issues the next item's first rows after its stores (below); the page ids
    // those rows need were requested in the last step: complete them before the stores, so that
    // nothing issued before the stores has to be waited for after them
    if constexpr (FOLD) BSR_DECODE_WAIT_VMCNT0();
    if (n < item.row_end - item.row_start) {
      const bool empty = !(l > 0.f);
      const float inv = empty ? 0.f : o_scale / l;
      const float lse = empty ? kNegInf : (m + log2f(l)) * kLn2;
      if (item.slot < 0) {
        uint16_t* op = O + orow * D + 4 * j;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const f32x4 v = oacc[db] * inv;
          *reinterpret_cast<u32x2*>(op + db * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
        if (j == 0) a.lse[orow] = lse;
      } else {
        const int64_t prow = (int64_t(item.slot) * a.Hk + hk) * a.Tq + n;  // row n of the tile
        if constexpr (FOLD) {  // read by whichever workgroup folds the tile: agent-scope stores
          const int32_t ob = int32_t(prow * D + 4 * j) * 4;
#pragma unroll
          for (int db = 0; db < DB; ++db)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, oacc[db] * inv), part_o_rs,
                                                   ob + 64 * db, 0, kAgentScope);
          if (j == 0)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse), part_lse_rs, int32_t(prow) * 4, 0,
                                                  kAgentScope);
        } else {
          float* pp = a.part_o + prow * D + 4 * j;
#pragma unroll
          for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(pp + db * 16) = oacc[db] * inv;
          if (j == 0) a.part_lse[prow] = lse;
        }
      }
    }

    // The last of a split tile's partial states folds the tile (the reduction of "FlashInfer:
    // Engineering a Customizable, Block-Sparse Attention Engine for LLM Inference Serving" §VIII.3
    // and §VIII.6, inside the attention kernel), per KV head: every wave that writes one of the
    // tile's states for its head waits until its stores are complete at agent scope and then counts
    // itself in; the wave that completes the count reads the tile's states in the plan's slot order
    // (KV order) and writes the final output, so the result does not depend on which workgroup
    // folded it, and returns the counter to zero for the next call.
    if constexpr (FOLD) {
      if (item_mi >= 0) {  // (uniform: all waves of the workgroup run the item)
        const int ns = fold_ns;
        const int* __restrict__ sl = a.mslots + fold_begin;
        const int sid_lane = fold_sid;
        if (more) {
          // the next item's first rows go out before the wait, so that their latency overlaps
          // the count and any fold; the wait then leaves exactly those 2 NL PD loads in flight
          // (loads and stores complete in issue order), so this item's stores are complete
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int h2 = 0; h2 < PD; ++h2)
            load_rows(kr0[h2], vr0[h2], next.kv_start + 16 * h2 + n, pre[h2], next.kv_end);
          have_rows = true;
          __builtin_amdgcn_sched_barrier(0);
          BSR_DECODE_WAIT_VMCNT(2 * NL * PD);
        } else {
          BSR_DECODE_WAIT_VMCNT0();
        }
        int32_t* ctr = a.arrive + int64_t(item_mi) * a.Hk + hk;
        int arrived = 0;
        if (lane == 0) arrived = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        arrived = __builtin_amdgcn_readfirstlane(arrived);
        if (arrived == ns - 1) {
          if (lane == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          // every lane folds 8 values of one row: lane c of a pass takes row c / (D / 8), values
          // 8 (c % (D / 8)) .. + 7, and issues the loads of kFoldSlots slots together, folded
          // with a running maximum: O = sum_k e^(lse_k - m) O_k / sum_k e^(lse_k - m)
          constexpr int CPR = D / 8;
          const int rows = item.row_end - item.row_start;
          for (int c0 = 0; c0 < rows * CPR; c0 += 64) {
            const int c = c0 + lane;
            const bool live = c < rows * CPR;
            const int r = live ? c / CPR : 0, col = 8 * (c % CPR);
            float mrun = kNegInf, den = 0.f;
            f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            for (int k0 = 0; k0 < ns; k0 += kFoldSlots) {
              // slot ids k0 .. k0 + kFoldSlots - 1 in lanes 0 .. kFoldSlots - 1 (the last id repeats
              // past the tile's end; those slots are skipped below)
              const int sid_k = k0 == 0 ? sid_lane : sl[min(k0 + lane % kFoldSlots, ns - 1)];
              float lk[kFoldSlots];
              f32x4 ok[kFoldSlots][2];
#pragma unroll
              for (int u = 0; u < kFoldSlots; ++u) {
                const int id = __shfl(sid_k, u, 64);
                const int32_t prow = (id * a.Hk + hk) * a.Tq + r;
                lk[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(part_lse_rs, prow * 4, 0, kAgentScope));
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2)
                  ok[u][h2] = __builtin_bit_cast(
                      f32x4, __builtin_amdgcn_raw_buffer_load_b128(part_o_rs, (prow * D + col + 4 * h2) * 4, 0,
                                                                   kAgentScope));
              }
#pragma unroll
              for (int u = 0; u < kFoldSlots; ++u) {
                if (k0 + u >= ns || lk[u] == kNegInf) continue;
                const float mn = fmaxf(mrun, lk[u]);
                const float so = expf(mrun - mn), w = expf(lk[u] - mn);
                den = den * so + w;
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) acc[h2] = acc[h2] * so + ok[u][h2] * w;
                mrun = mn;
              }
            }
            if (live) {
              const bool empty = !(den > 0.f);
              const float inv = empty ? 0.f : 1.f / den;
              const int row = item.row_start + r;
              const int64_t orow_r = int64_t(item.q_start + row / g) * a.Hq + hk * g + row % g;
              const f32x4 v0 = acc[0] * inv, v1 = acc[1] * inv;
              *reinterpret_cast<u32x4*>(O + orow_r * D + col) =
                  u32x4{pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]), pack_bf16x2(v1[0], v1[1]),
                        pack_bf16x2(v1[2], v1[3])};
              if (col == 0) a.lse[orow_r] = empty ? kNegInf : mrun + logf(den);
            }
          }
        }
      }
    }
  }
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(tk + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == int(gridDim.x) - 1) {  // every workgroup has drawn its last ticket
      __hip_atomic_store(tk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(tk + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

bool decode_bf16_supported(int d, int g, int Tq) {
  return (d == 64 || d == 128) && g >= 1 && g <= 16 && g <= Tq;
}

bool decode_bf16_tiles(int d, int g, int Tq) { return (d == 64 || d == 128) && g >= 1 && Tq <= 16; }

// waves per workgroup: the largest divisor of H_kv up to kDecodeWaves, so that every wave of a
// workgroup has a KV head (they all join the ticket barriers)
int decode_bf16_waves_per_block(int Hk) {
  for (int wv = kDecodeWaves; wv > 1; --wv)
    if (Hk % wv == 0) return wv;
  return 1;
}

int decode_bf16_blocks_per_worker(int Hk) {
  const int wv = decode_bf16_waves_per_block(Hk);
  return (Hk + wv - 1) / wv;
}

int decode_bf16_blocks_per_cu(int d, int Hk) {
  const int wv = decode_bf16_waves_per_block(Hk);
  int nb = 1;
  hipError_t e = hipErrorInvalidValue;
  if (d == 64)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_decode_bf16_kernel<64, false, false, true, false>, 64 * wv,
                                                     wv * decode_vs_bytes<64>());
  if (d == 128)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_decode_bf16_kernel<128, false, false, true, false>, 64 * wv,
                                                     wv * decode_vs_bytes<128>());
  return (e == hipSuccess && nb > 0) ? nb : 1;
}

// The affine (contiguous-cache) instantiation exists for the plain bf16 kernel; the other
// variants read the identity table that an affine plan stores like any other.
template <int D, bool KV8, bool FOLD>
static void launch_cap(const RunArgs& a, dim3 grid, int waves, hipStream_t s) {
  const size_t lds = size_t(waves) * decode_vs_bytes<D>();
  if (a.soft_cap > 0.f)
    hipLaunchKernelGGL((attn_decode_bf16_kernel<D, true, KV8, FOLD, false>), grid, dim3(64 * waves), lds, s, a);
  else if (!KV8 && a.affine)
    hipLaunchKernelGGL((attn_decode_bf16_kernel<D, false, KV8, FOLD, !KV8>), grid, dim3(64 * waves), lds, s, a);
  else
    hipLaunchKernelGGL((attn_decode_bf16_kernel<D, false, KV8, FOLD, false>), grid, dim3(64 * waves), lds, s, a);
}

// Workgroups that stay resident together on the current device (per head group); items are taken
// from the ticket list, so the grid needs no more workgroups than that, whatever the plan's C.
static int decode_resident_blocks(int d, int Hk) {
  static int cached[2][65] = {};
  const int di = d == 64 ? 0 : 1, hi = Hk < 64 ? Hk : 64;
  if (!cached[di][hi]) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return INT32_MAX;
    cached[di][hi] = cus * decode_bf16_blocks_per_cu(d, Hk);
  }
  return cached[di][hi];
}

hipError_t launch_decode_bf16(const RunArgs& a, bool kv_e4m3, hipStream_t s) {
  const int waves = decode_bf16_waves_per_block(a.Hk);
  const dim3 grid(std::min(a.C, decode_resident_blocks(a.d, a.Hk)), decode_bf16_blocks_per_worker(a.Hk));
  if (a.d == 64 && kv_e4m3 && a.fold_in_kernel) launch_cap<64, true, true>(a, grid, waves, s);
  else if (a.d == 64 && kv_e4m3) launch_cap<64, true, false>(a, grid, waves, s);
  else if (a.d == 64 && a.fold_in_kernel) launch_cap<64, false, true>(a, grid, waves, s);
  else if (a.d == 64) launch_cap<64, false, false>(a, grid, waves, s);
  else if (a.d == 128 && kv_e4m3 && a.fold_in_kernel) launch_cap<128, true, true>(a, grid, waves, s);
  else if (a.d == 128 && kv_e4m3) launch_cap<128, true, false>(a, grid, waves, s);
  else if (a.d == 128 && a.fold_in_kernel) launch_cap<128, false, true>(a, grid, waves, s);
  else if (a.d == 128) launch_cap<128, false, false>(a, grid, waves, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bsr
