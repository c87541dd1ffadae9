// bf16 tiled attention on gfx950 matrix cores: ragged (causal) prefill over a paged
// KV cache, with GQA-packed query tiles.
//
// Data path ("sparse select, dense compute": "FlashInfer: Engineering a
// Customizable, Block-Sparse Attention Engine for LLM Inference Serving" §IV.2 and
// §V.4; "FlashInfer 原理" §⑥): the rows of a 64-token KV tile are looked up through
// the page table (eq. 7 of "FlashInfer: Making Attention Fit the Serving Workload")
// and copied from HBM straight into LDS by 16-byte LDS-DMA loads
// (global_load_lds_dwordx4), in an order the matrix instructions read without bank
// conflicts; after staging the products are ordinary dense MFMA tiles.  A query tile
// holds T_q packed rows of one KV head (row r -> position floor(r / g), head
// g * h_kv + r mod g, eq. 3 of the review), so every staged KV tile serves all g query
// heads of the group.
//
// LDS layout: four arrays, two K slots and two V slots, each one 64-token tile of K (or V)
// as 4 token groups (16 tokens) x D/32 column groups (32 head-dim values) of 1 KB fragments,
// 64 lanes x 16 bytes:
//   K fragment (a, b): byte 16 L holds K[16a + L%16][32b + 8(L/16) .. +8]
//   V fragment (a, b): byte 16 L holds V[16a + t][32b + 8c .. +8], c = L/16,
//                      t = (L%16) xor s(c), s(c) = 8(c%2) + 4(c/2)
// Every DMA instruction reads 64 contiguous bytes of 16 token rows.  The V swizzle makes every
// ds_read_b64_tr_b16 (32 lanes x 8 bytes per LDS cycle on gfx950's 64 banks) touch each bank
// once, for both matrix shapes below; K reads are linear or one 256-byte row apart.
//
// Large query tiles (more than 64 packed rows) use v_mfma_f32_32x32x16_bf16 (on gfx950 it
// sustains about twice the rate of the 16x16x32 shape), one 32-row block per wave, and a
// software pipeline over the KV tiles: while the matrix cores compute the scores of tile i+1,
// the vector ALUs run the softmax of tile i; then P.V of tile i runs.  Per wave:
//   S^T[token][row] = sum_k K[token][k] Q[row][k]   (A = K, B = Q^T kept in registers)
//     lane L holds, for row L%32, tokens 8(i/4) + 4(L/32) + i%4, i = 0..15, of a
//     32-token block
//   online softmax per row in log2 units ("FlashInfer: Engineering ...", §II.2); the
//     reference maximum is raised only when a score exceeds it by more than 8 (so
//     p <= 256), which keeps the result exact (numerator and denominator share the
//     reference) and makes the rescale of the accumulator rare
//   O^T[d][row] += sum_token V^T[d][token] P^T[token][row]: B = P^T is the score
//     accumulator converted to bf16 in place (items 8k..8k+7 form one 16-token k-block),
//     A = V^T from two transposing reads per k-block, with the same token order.
// K and V have their own rings with a barrier each per tile, so each is fetched 1.5 tiles
// ahead of its use; the waits name the exact number of younger loads that may still be in
// flight.
// Query tiles of 33-64 rows use the same 32x32 products on two waves per row block (each
// takes half of every KV tile); tiles of at most 32 rows (decode-like and short requests,
// the composable prefix level) use the 16x16x32 shape with 16-row blocks.  These smaller
// shapes use a plain two-stage loop.
//
// Every wave computes all of its row blocks, including absent ones at the end of a
// request (zero queries, never written), so the products carry no branches.  When a
// tile has fewer row blocks than waves, waves also split the tile's tokens and their
// states are combined at the end of the item with the merge of eq. 6 (§3.2 of the
// review).
//
// Variants ("FlashInfer 原理" §⑧; eq. 8 of the review) run in separate instantiations (VAR): the
// sliding window in both kernels, the soft cap and custom masks in the 4-wave one.  The soft cap turns each score s into
// (c / sm_scale) tanh(sm_scale s / c) before the mask (the softmax then multiplies by
// sm_scale log2(e) as usual), a sliding window adds a per-row lower bound to the mask, and a
// custom mask is read bit by bit for every block (its loads are ordinary vector loads, so the
// compiler's wait for them also waits for the tile loads in flight: masked runs give up the
// prefetch depth).
#include <climits>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace bsr {

namespace {

constexpr int kTileKV = 64;  // tokens per staged KV tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kThreads2 = 128;  // workgroup of the 128-row shape: two waves of 512 VGPRs
constexpr float kRescaleMargin = 8.f;  // log2 units
constexpr float kMFloor = -1e30f;      // initial reference of the 32-row shapes (log2 units)
constexpr int kPageWindow = 2048;      // page ids staged in LDS per workgroup

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int D>
struct PF {
  static constexpr int KB = D / 32;           // 32-wide column groups per row
  static constexpr int FRAG = 1024;           // 64 lanes x 16 bytes
  static constexpr int TILE = 4 * KB * FRAG;  // K (or V) of 64 tokens
  static constexpr int COMB16 = 16 * (D + 2) * 4;  // combine area of one 16-row wave
  static constexpr int COMB32 = 32 * (D + 2) * 4;  // combine area of one 32-row wave
  static constexpr int SLOT = TILE > COMB32 ? TILE : COMB32;  // bytes of one LDS array
  static_assert(2 * COMB16 <= SLOT, "two 16-row combine areas must fit in one array");
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// LDS-typed pointers: slot arithmetic stays in 32-bit LDS addresses and every access is a
// ds_* instruction, also where a slot is chosen at run time
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) int32_t lds_i32;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

// The workgroup's LDS: four SLOT-byte arrays (K and V of two 64-token tiles; the pipelined
// path splits each into two 32-token slots) and the page-id window.
template <int D>
struct Slots {
  lds_u8* base;
  __device__ __forceinline__ lds_u8* k0() const { return base; }
  __device__ __forceinline__ lds_u8* k1() const { return base + PF<D>::SLOT; }
  __device__ __forceinline__ lds_u8* v0() const { return base + 2 * PF<D>::SLOT; }
  __device__ __forceinline__ lds_u8* v1() const { return base + 3 * PF<D>::SLOT; }
  __device__ __forceinline__ lds_i32* table() const { return reinterpret_cast<lds_i32*>(base + 4 * PF<D>::SLOT); }
  // the next work item's record, fetched during the current item
  __device__ __forceinline__ lds_i32* rec() const {
    return reinterpret_cast<lds_i32*>(base + 4 * PF<D>::SLOT + 4 * kPageWindow);
  }
  static constexpr int BYTES = 4 * PF<D>::SLOT + 4 * kPageWindow + sizeof(ItemRec);
};

// The next work item's record, fetched while the current item starts: lane l of the first
// kRecWords threads loads word l before the current item issues its first tile loads, and
// stores it to the record slot in LDS once the item's prologue has waited for its own loads, so
// a new item starts with an LDS read instead of dependent global loads.
constexpr int kRecWords = int(sizeof(ItemRec) / 4);
struct RecFetch {
  int32_t word = 0;
  bool valid = false;  // uniform: there is a next item
  __device__ __forceinline__ void load(const ItemRec* next, bool has_next) {
    valid = has_next;
    if (has_next && threadIdx.x < kRecWords) word = reinterpret_cast<const int32_t*>(next)[threadIdx.x];
  }
  __device__ __forceinline__ void store(lds_i32* rec) const {
    if (valid && threadIdx.x < kRecWords) rec[threadIdx.x] = word;
  }
};
__device__ __forceinline__ ItemRec read_rec(const lds_i32* rec) {
  int32_t w[kRecWords];
#pragma unroll
  for (int i = 0; i < kRecWords; ++i) w[i] = __builtin_amdgcn_readfirstlane(rec[i]);
  ItemRec r;
  __builtin_memcpy(&r, w, sizeof(ItemRec));
  return r;
}
// The request fields the kernels use, from the item record (the custom-mask offset, needed only
// with a mask, from the request record)
__device__ __forceinline__ ReqRec req_of(const RunArgs& a, const ItemRec& it);

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  bf16x2 r;
  r[0] = static_cast<__bf16>(a);
  r[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + the two bf16 values of a packed pair (v_dot2_f32_bf16 against (1, 1)): the row sum
// adds the same rounded weights that P.V multiplies, one instruction per pair
__device__ __forceinline__ float sum_pair(uint32_t pair, float acc) {
  const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), ones, acc, false);
}

// max / sum of the values held by lanes l and l ^ 32, through v_permlane32_swap (no LDS
// round trip).  The swap exchanges the upper half of its first operand with the lower half of
// its second, so with both operands x every lane ends up holding x[l] and x[l ^ 32].
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const unsigned a = r[0], b = r[1];
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const unsigned a = r[0], b = r[1];
  return __uint_as_float(a) + __uint_as_float(b);
}
// the same for lanes l and l ^ 16 (v_permlane16_swap exchanges odd 16-lane rows of its first
// operand with even rows of its second)
__device__ __forceinline__ float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const unsigned a = r[0], b = r[1];
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const unsigned a = r[0], b = r[1];
  return __uint_as_float(a) + __uint_as_float(b);
}

__device__ __forceinline__ s16x4 tr_read(const lds_u8* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p));
}

__device__ __forceinline__ bf16x8 cat(s16x4 lo, s16x4 hi) {
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// row swizzle of the 16-byte column chunk c16 (0..3) inside a V fragment
__device__ __forceinline__ int v_swz(int c16) { return 8 * (c16 & 1) + 4 * (c16 >> 1); }

// byte offset, inside a V fragment, of the 8-byte chunk c (head-dim 4c .. 4c+3 of the
// fragment's 32 columns) of token t (0..15)
__device__ __forceinline__ int v_chunk(int t, int c) {
  const int c16 = c >> 1;
  return 16 * (16 * c16 + (t ^ v_swz(c16))) + 8 * (c & 1);
}

// Plan records are the same for the whole workgroup: read them once and keep every field in
// a scalar register, so everything derived from them is uniform (scalar branches, no
// per-lane copies).
template <typename T>
__device__ __forceinline__ T uniform_load(const T* p) {
  static_assert(sizeof(T) % 4 == 0, "records of 32-bit fields");
  int32_t w[sizeof(T) / 4];
  __builtin_memcpy(w, p, sizeof(T));
#pragma unroll
  for (unsigned i = 0; i < sizeof(T) / 4; ++i) w[i] = __builtin_amdgcn_readfirstlane(w[i]);
  T v;
  __builtin_memcpy(&v, w, sizeof(T));
  return v;
}

__device__ __forceinline__ ReqRec req_of(const RunArgs& a, const ItemRec& it) {
  ReqRec r;
  r.q_start = it.q_start;
  r.q_len = it.q_len;
  r.page_start = it.page_start;
  r.kv_len = it.kv_len;
  r.tok_start = 0;
  r.pad = 0;
  r.mask_off = a.mask ? uniform_load(a.req + it.req).mask_off : 0;
  return r;
}

// Page-size classes the kernels are compiled for: any size (division), a power of two (shift
// and mask), or a power of two that divides 32 (then a token's offset inside its page is the
// same in every 32-token tile of an item, and its page number advances by 32 / P per tile).
constexpr int kPageAny = 0, kPagePow2 = 1, kPageDiv32 = 2;

// Token -> page lookups (eq. 7 of "FlashInfer: Making Attention Fit the Serving Workload").
// A window of up to kPageWindow entries of the request's page list is staged in LDS, so the
// lookups inside the tile loops are LDS reads and the only vector-memory loads in flight there
// are the tile DMAs.  POW2: the page size is a power of two (shift and mask).
constexpr int kRefillBatch = 4;  // page-id loads in flight per thread during a window refill

template <bool POW2>
struct Paging {
  const int32_t* indices;  // the request's page list starts at indices + page_start
  lds_i32* table;          // LDS window: table[j] = page id of request page base + j
  int32_t page_start, P, p_shift, Hk, hk, kv_end;
  int32_t base;  // first request page held in the window
  __device__ __forceinline__ int page_no(int t) const {
    const int tc = min(t, kv_end - 1);
    return POW2 ? (tc >> p_shift) : tc / P;
  }
  __device__ __forceinline__ int32_t page_of(int t) const { return table[page_no(t) - base]; }
  // first element of token t's row for this KV head, t clamped to the chunk
  template <int D>
  __device__ __forceinline__ int64_t row(int t, int32_t page) const {
    const int tc = min(t, kv_end - 1);
    const int off = POW2 ? (tc & (P - 1)) : tc - (tc / P) * P;
    // page * (P Hk D) + (off Hk + hk) D as one unsigned 32x32 -> 64-bit multiply-add (page
    // ids are non-negative; the planner keeps P Hk D below 2^31)
    return int64_t(uint64_t(uint32_t(page)) * uint32_t(P * Hk * D) + uint32_t((off * Hk + hk) * D));
  }
  // (Re)fill the window so it holds the pages of tokens [lo, hi]; lo and hi are uniform and
  // every thread of the workgroup (NTH of them) calls this (it synchronises the workgroup
  // when it refills).
  // At an item's start (START) the loads of the refill are issued kRefillBatch per thread before
  // their values are stored, so a window of up to NTH * kRefillBatch entries costs one memory
  // round trip there; inside the tile loops, where a refill is rare (an item longer than the
  // window) and registers are scarce, one entry per thread at a time.
  template <int NTH = kThreads, bool START = false>
  __device__ __forceinline__ void cover(int lo, int hi) {
    const int plo = page_no(lo), phi = page_no(hi);
    if (plo >= base && phi < base + kPageWindow) return;
    __syncthreads();  // nobody reads the old window any more
    base = plo;
    const int cnt = min(kPageWindow, page_no(kv_end - 1) - plo + 1);
    const int32_t* __restrict__ src = indices + page_start + plo;
    if constexpr (START) {
      // (cnt >= 1: page_no clamps to the chunk's last token; a load past cnt re-reads entry
      // cnt - 1, so the first batch is straight-line code and none of its loads waits for another)
      auto batch = [&](int j0) {
        int32_t v[kRefillBatch];
#pragma unroll
        for (int u = 0; u < kRefillBatch; ++u) v[u] = src[min(j0 + u * NTH + int(threadIdx.x), cnt - 1)];
#pragma unroll
        for (int u = 0; u < kRefillBatch; ++u) {
          const int j = j0 + u * NTH + int(threadIdx.x);
          if (j < cnt) table[j] = v[u];
        }
      };
      batch(0);
      for (int j0 = NTH * kRefillBatch; j0 < cnt; j0 += NTH * kRefillBatch) batch(j0);
    } else {
      for (int j = threadIdx.x; j < cnt; j += NTH) table[j] = src[j];
    }
    __syncthreads();
  }
};

// tokens (within the wave's 16-token group) carried by this lane in K / V fragments
__device__ __forceinline__ int k_dma_token(int lane) { return lane & 15; }
__device__ __forceinline__ int v_dma_token(int lane) { return (lane & 15) ^ v_swz(lane >> 4); }

// pages of the tokens this lane carries in the K / V fragments of the tile starting at t0
template <class PG>
__device__ __forceinline__ int32_t k_page(const PG& pgn, int t0) {
  return pgn.page_of(t0 + (threadIdx.x >> 6) * 16 + k_dma_token(threadIdx.x & 63));
}
template <class PG>
__device__ __forceinline__ int32_t v_page(const PG& pgn, int t0) {
  return pgn.page_of(t0 + (threadIdx.x >> 6) * 16 + v_dma_token(threadIdx.x & 63));
}

// KB LDS-DMA loads (global_load_lds_dwordx4) of one wave: load b reads 16 bytes per lane
// from src + 64 b bytes and writes them lane-linearly to LDS fragment b (1 KB apart) starting
// at lds.  The instruction offset (64 b) applies to the LDS address as well as the global one,
// so M0 holds lds + b (1024 - 64) for load b.  The M0 values are computed outside the asm and
// set with s_mov_b32, which leaves SCC alone (the asm also declares SCC clobbered, so no
// compare may live across it).  Written as one asm block so the compiler does not track these
// loads: every wait for them is explicit (BSR_WAIT_VMCNT before the barrier that publishes a
// slot), and no read of one slot waits for the loads still filling another.
template <int KB>
__device__ __forceinline__ void dma_fragments(const uint16_t* src, const lds_u8* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)));
  static_assert(KB == 1 || KB == 2 || KB == 4, "one, two or four fragments");
  constexpr uint32_t kStep = 1024 - 64;
  uint32_t saved;  // M0 is restored afterwards: the compiler treats it as reserved
  if constexpr (KB == 1) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(m0)
        : "memory", "scc");
  } else if constexpr (KB == 2) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off offset:64\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(m0), "s"(m0 + kStep)
        : "memory", "scc");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off offset:64\n\t"
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off offset:128\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off offset:192\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(m0), "s"(m0 + kStep), "s"(m0 + 2 * kStep), "s"(m0 + 3 * kStep)
        : "memory", "scc");
  }
}

// The K and V batches of one steady pipeline step in one asm block (NF = 2 or 4 fragments each):
// ksrc / vsrc are this lane's 16-byte sources of fragment 0, kdst / vdst the wave's first LDS
// fragments (uniform).  M0 is written straight from the base plus the fragment's offset
// b (1024 - 64), and saved and restored once for the whole block.  Same loads, in the same order,
// as dma_fragments<NF> for K followed by dma_fragments<NF> for V.
#define BSR_DMA_FRAG(src, base, b) \
  "s_add_u32 m0, " base ", " #b " * 960\n\ts_nop 0\n\tglobal_load_lds_dwordx4 " src ", off offset:" #b " * 64\n\t"
template <int NF>
__device__ __forceinline__ void dma_kv(const uint16_t* ksrc, uint32_t kdst, const uint16_t* vsrc, uint32_t vdst) {
  static_assert(NF == 1 || NF == 2 || NF == 4, "one, two or four fragments per batch");
  static_assert(1024 - 64 == 960, "M0 step between fragments");
  uint32_t saved;
  if constexpr (NF == 4) {
    asm volatile("s_mov_b32 %0, m0\n\t"
                 BSR_DMA_FRAG("%1", "%3", 0) BSR_DMA_FRAG("%1", "%3", 1) BSR_DMA_FRAG("%1", "%3", 2)
                 BSR_DMA_FRAG("%1", "%3", 3) BSR_DMA_FRAG("%2", "%4", 0) BSR_DMA_FRAG("%2", "%4", 1)
                 BSR_DMA_FRAG("%2", "%4", 2) BSR_DMA_FRAG("%2", "%4", 3)
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(ksrc), "v"(vsrc), "s"(kdst), "s"(vdst)
                 : "memory", "scc");
  } else if constexpr (NF == 2) {
    asm volatile("s_mov_b32 %0, m0\n\t"
                 BSR_DMA_FRAG("%1", "%3", 0) BSR_DMA_FRAG("%1", "%3", 1)
                 BSR_DMA_FRAG("%2", "%4", 0) BSR_DMA_FRAG("%2", "%4", 1)
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(ksrc), "v"(vsrc), "s"(kdst), "s"(vdst)
                 : "memory", "scc");
  } else {
    asm volatile("s_mov_b32 %0, m0\n\t"
                 BSR_DMA_FRAG("%1", "%3", 0) BSR_DMA_FRAG("%2", "%4", 0)
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(ksrc), "v"(vsrc), "s"(kdst), "s"(vdst)
                 : "memory", "scc");
  }
}
#undef BSR_DMA_FRAG


// LDS-DMA loads of the K (V) half of the 64-token tile at t0 into one array: wave w loads
// token group w, D/32 fragments; `page` comes from k_page (v_page) one step earlier
template <int D, class PG>
__device__ __forceinline__ void issue_k(lds_u8* slot, const PG& pgn, int t0, int32_t page,
                                        const uint16_t* K) {
  constexpr int KB = PF<D>::KB;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  dma_fragments<KB>(K + pgn.template row<D>(t0 + w * 16 + k_dma_token(lane), page) + 8 * (lane >> 4),
                    slot + w * KB * PF<D>::FRAG);
}
template <int D, class PG>
__device__ __forceinline__ void issue_v(lds_u8* slot, const PG& pgn, int t0, int32_t page,
                                        const uint16_t* V) {
  constexpr int KB = PF<D>::KB;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  dma_fragments<KB>(V + pgn.template row<D>(t0 + w * 16 + v_dma_token(lane), page) + 8 * (lane >> 4),
                    slot + w * KB * PF<D>::FRAG);
}

// O^T += V^T P^T on the matrix cores with the accumulator held in AGPRs (the 128-row shape
// keeps its 128 accumulator registers there and everything the vector ALUs touch in VGPRs).
// The compiler does not see inside the asm, so reads of the accumulator by other
// instructions wait for the product explicitly (acc_settle).
__device__ __forceinline__ void mfma_acc_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last accumulator product and any other access to the accumulators
// (at least the latency of a 16-pass product).
__device__ __forceinline__ void acc_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// Empty volatile asm that reads and rewrites its operands: the values must exist at this
// point of the program, so the code computing them cannot sink below it.
__device__ __forceinline__ void pin(f32x16& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(u32x4 (&v)[2]) { asm volatile("" : "+v"(v[0]), "+v"(v[1])); }

// Instruction classes of the scheduling-group builtin, and an interleave of NM matrix
// instructions with the LDS reads that feed them (AHEAD issued first, then PER after each
// matrix instruction) and VALU vector-ALU instructions after each, so that independent vector
// work issues while the matrix core is busy.
constexpr int kSgValu = 0x002, kSgMfma = 0x008, kSgDsRead = 0x100;
template <int NM, int AHEAD, int PER, int VALU>
__device__ __forceinline__ void sched_mfma_interleave() {
  __builtin_amdgcn_sched_group_barrier(kSgDsRead, AHEAD, 0);
#pragma unroll
  for (int j = 0; j < NM; ++j) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, PER, 0);
    __builtin_amdgcn_sched_group_barrier(kSgValu, VALU, 0);
  }
}

// Wait until at most n vector-memory loads of this wave are in flight (loads complete in
// order), leaving LDS and export counters alone.  n must be a compile-time constant.
#define BSR_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// LDS-DMA accounting of the two pipelined shapes.  Step j of the stream reads K(j+1) and V(j-1);
// in step j a wave issues one batch of NF loads of K(j + kKAhead), then one of V(j + kVAhead), so
// the loads of every tile go out kIssueToUseSteps steps before the barrier that publishes it.  At
// that barrier's wait, the batches younger than the ones needed are those of the steps in between:
// at most kMaxBatchesInFlight batches may stay in flight.  vmcnt counts every vector-memory
// instruction of the wave, in issue order; nothing else in the step loop touches vector memory
// (page ids come from the LDS window, and a window refill waits for its own loads, hence for every
// older load too), so the limits below count exactly these batches.
constexpr int kIssueToUseSteps = 3;
constexpr int kKAhead = kIssueToUseSteps + 1, kVAhead = kIssueToUseSteps - 1;
constexpr int kDmaBatchesPerStep = 2;
constexpr int kMaxBatchesInFlight = kDmaBatchesPerStep * (kIssueToUseSteps - 1);
static_assert(kKAhead - 1 == kIssueToUseSteps && kVAhead + 1 == kIssueToUseSteps,
              "step j reads K(j+1) and V(j-1): both issued kIssueToUseSteps steps earlier");
static_assert(kMaxBatchesInFlight == kDmaBatchesPerStep * (kIssueToUseSteps - 1),
              "the batches of the steps between a tile's issue and its barrier");

// Batches issued in the steps between the needed ones and step j (steps j - kIssueToUseSteps + 1
// .. j - 1) that exist in an item of n tiles (the last steps skip loads past the end).
__device__ __forceinline__ int batches_in_between(int j, int n) {
  int c = 0;
#pragma unroll
  for (int s = 1; s < kIssueToUseSteps; ++s) c += (j - s + kKAhead < n) + (j - s + kVAhead < n);
  return c;
}

// Wait until at most nb (0 .. kMaxBatchesInFlight) batches of NF loads are in flight.
template <int NF>
__device__ __forceinline__ void wait_dma_batches(int nb) {
  static_assert(kMaxBatchesInFlight * NF <= 63, "the vmcnt field holds 0 .. 63");
  static_assert(kMaxBatchesInFlight <= 4, "one case per batch count");
  switch (nb) {
    case 4: BSR_WAIT_VMCNT(4 * NF); break;
    case 3: BSR_WAIT_VMCNT(3 * NF); break;
    case 2: BSR_WAIT_VMCNT(2 * NF); break;
    case 1: BSR_WAIT_VMCNT(NF); break;
    default: BSR_WAIT_VMCNT(0); break;
  }
}

// The plain double-buffered tile loop of the smaller shapes: compute(k_slot, v_slot, t0) is
// called once per 64-token tile while the next tile's DMA is in flight.
template <int D, class PG, typename F>
__device__ __forceinline__ void tile_loop(PG& pgn, int kv_start, int kv_end, const Slots<D>& s, const uint16_t* K,
                                          const uint16_t* V, F&& compute) {
  const int ntiles = (kv_end - kv_start + kTileKV - 1) / kTileKV;
  __syncthreads();  // LDS free (previous item finished, including its combine)
  pgn.base = -kPageWindow;  // nothing staged for this item yet
  pgn.template cover<kThreads, true>(kv_start, kv_start + 2 * kTileKV - 1);
  int32_t pk = k_page(pgn, kv_start), pv = v_page(pgn, kv_start);
  issue_k<D>(s.k0(), pgn, kv_start, pk, K);
  issue_v<D>(s.v0(), pgn, kv_start, pv, V);
  pk = k_page(pgn, kv_start + kTileKV);
  pv = v_page(pgn, kv_start + kTileKV);
  BSR_WAIT_VMCNT(0);  // this wave's DMA has landed
  __syncthreads();    // ... and every wave's
  for (int ti = 0; ti < ntiles; ti += 2) {
    const int t0 = kv_start + ti * kTileKV;
    pgn.cover(t0 + 2 * kTileKV, t0 + 4 * kTileKV - 1);
    if (ti + 1 < ntiles) {
      issue_k<D>(s.k1(), pgn, t0 + kTileKV, pk, K);
      issue_v<D>(s.v1(), pgn, t0 + kTileKV, pv, V);
      pk = k_page(pgn, t0 + 2 * kTileKV);
      pv = v_page(pgn, t0 + 2 * kTileKV);
    }
    compute(static_cast<const lds_u8*>(s.k0()), static_cast<const lds_u8*>(s.v0()), t0);
    BSR_WAIT_VMCNT(0);
    __syncthreads();
    if (ti + 1 < ntiles) {
      if (ti + 2 < ntiles) {
        issue_k<D>(s.k0(), pgn, t0 + 2 * kTileKV, pk, K);
        issue_v<D>(s.v0(), pgn, t0 + 2 * kTileKV, pv, V);
        pk = k_page(pgn, t0 + 3 * kTileKV);
        pv = v_page(pgn, t0 + 3 * kTileKV);
      }
      compute(static_cast<const lds_u8*>(s.k1()), static_cast<const lds_u8*>(s.v1()), t0 + kTileKV);
      BSR_WAIT_VMCNT(0);
      __syncthreads();
    }
  }
}

// Online-softmax reference update for one row held by this lane (identical across the
// lanes that share the row): raise the reference only past the margin; returns the
// rescale factor (1 when the reference stays).
__device__ __forceinline__ float raise_reference(float& m, float mx_scaled, bool& any) {
  const bool raise = mx_scaled > m + kRescaleMargin;
  any = __ballot(raise) != 0;
  if (!any) return 1.f;
  const float mnew = raise ? mx_scaled : m;
  const float corr = fast_exp2(m - (mnew == kNegInf ? 0.f : mnew));
  m = mnew;
  return corr;
}

// ---------------------------------------------------------------------------------
// Large query tiles: 32-row blocks on v_mfma_f32_32x32x16_bf16; every wave takes one
// 32-token block per tile.
// PIPE: more than 64 rows, one row block per wave, software-pipelined over 32-token tiles.
// Otherwise (33-64 rows): two row blocks, each shared by two waves that take the two
// 32-token halves of every 64-token tile of the plain loop.
// ---------------------------------------------------------------------------------
// Per-row state of the variants: the first key the sliding window shows this row (INT_MIN
// without a window), the largest such key over the item's rows (uniform; KV blocks that
// start before it need the lower-bound test), the soft cap as S -> k1 tanh(k2 S), and the
// first bit of this row in a custom mask (-1: no mask, or an absent row).
struct VarRow {
  int lo = INT_MIN, max_lo = INT_MIN;
  float k1 = 0.f, k2 = 0.f;
  int64_t mrow = -1;
  int64_t last_byte = 0;  // last byte holding bits of this request (custom mask)
  bool masked = false;    // a custom mask is given (uniform): every block is tested
  __device__ __forceinline__ VarRow(const RunArgs& a, const ItemRec& item, const ReqRec& rq, int row_pos,
                                    bool row_ok) {
    if (a.mask) {
      masked = true;
      if (row_ok) mrow = rq.mask_off + int64_t(row_pos) * rq.kv_len;
      last_byte = (rq.mask_off + int64_t(rq.q_len) * rq.kv_len - 1) >> 3;
    }
    if (a.window_left >= 0) {
      const int base = rq.kv_len - rq.q_len - a.window_left;
      lo = base + row_pos;
      max_lo = __builtin_amdgcn_readfirstlane(base + (item.row_end - 1) / a.g);
    }
    if (a.soft_cap > 0.f) {
      k1 = a.soft_cap / a.sm_scale;
      k2 = a.sm_scale / a.soft_cap;
    }
  }
  __device__ __forceinline__ float cap(float s) const { return k1 * fast_tanh(k2 * s); }
  // With a custom mask: this row's bits of keys tb .. tb + 31 (bit k for key tb + k), from the
  // five bytes that hold them; each byte index is clamped to the request's last byte, so every
  // load is inside the mask (clamped bytes only serve keys past the row, which keeps_at drops).
  __device__ __forceinline__ uint32_t window(const uint8_t* __restrict__ mask, int tb) const {
    if (!masked) return 0u;  // uniform
    const int64_t bit0 = (mrow >= 0 ? mrow : 0) + tb;
    const int64_t b0 = bit0 >> 3;
    uint64_t w = 0;
#pragma unroll
    for (int q = 0; q < 5; ++q) w |= uint64_t(mask[min(b0 + q, last_byte)]) << (8 * q);
    return uint32_t(w >> (bit0 & 7));
  }
  // whether key tok = tb + k takes part: inside [lo, lim) and, with a custom mask, its bit in
  // win = window(mask, tb) set; combined without a branch (the loads happen in window())
  __device__ __forceinline__ bool keeps_at(uint32_t win, int k, int tok, int lim) const {
    const bool in = tok < lim && tok >= lo;
    if (!masked) return in;  // uniform
    return in & (mrow >= 0) & ((win >> k) & 1u);
  }
};

template <int D, bool PIPE, int PG, bool VAR>
__device__ __forceinline__ void prefill_item32(const RunArgs& a, const ItemRec& item, const ReqRec& rq, int hk,
                                               const Slots<D>& sl) {
  constexpr int KB = PF<D>::KB, FRAG = PF<D>::FRAG;
  constexpr int KS16 = D / 16;  // 16-deep k-steps of the score product
  constexpr int N_KS = PIPE ? 1 : 2;
  constexpr int N_RG = kWaves / N_KS;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r32 = lane & 31, h = lane >> 5;
  constexpr bool POW2 = PG != kPageAny;
  // row block; 32-token block within a tile (the pipelined shape has one row block per wave)
  const int rg = PIPE ? wave : wave % N_RG, ks = PIPE ? 0 : wave / N_RG;
  const int nrows = item.row_end - item.row_start;
  const float c = a.sm_scale * kLog2e;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  const int kv_end = item.kv_end;
  Paging<POW2> pgn{a.indices, sl.table(), rq.page_start, a.P, a.p_shift, a.Hk, hk, kv_end, -kPageWindow};

  // this lane's query row: block rg, row r32
  const int r = item.row_start + rg * 32 + r32;
  const bool rb_on = rg * 32 < nrows;
  const bool row_ok = r < item.row_end;
  const int row_pos = r / a.g, row_hq = hk * a.g + r % a.g;
  const int lim = (a.causal && row_ok) ? min(kv_end, rq.kv_len - rq.q_len + row_pos + 1) : kv_end;
  const VarRow var(a, item, rq, row_pos, row_ok);
  bf16x8 qb[KS16];
  {
    const uint16_t* qp = Q + (int64_t(rq.q_start + row_pos) * a.Hq + row_hq) * D + 8 * h;
#pragma unroll
    for (int k = 0; k < KS16; ++k) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4*>(qp + 16 * k);
      qb[k] = __builtin_bit_cast(bf16x8, v);
    }
  }
  int min_lim = kv_end;  // tiles ending before the smallest visible end need no mask
  if (a.causal) min_lim = min(kv_end, rq.kv_len - rq.q_len + item.row_start / a.g + 1);
  min_lim = __builtin_amdgcn_readfirstlane(min_lim);  // uniform: the mask test is a scalar branch

  // Running reference in log2 units.  It starts at a finite floor far below any score, so the
  // exponent S c - m is -inf for masked scores and finite otherwise, with no special case;
  // a row that saw no visible key keeps l = 0 and is written as the empty state.
  float m = kMFloor, l = 0.f, corr = 1.f;
  f32x16 oacc[KB];
#pragma unroll
  for (int b = 0; b < KB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[b][i] = 0.f;

  // K fragment position of this lane for k-step k (token r32 of the 32-token block, half h)
  const int k_pos = 16 * ((r32 & 15) + 16 * h);  // + 512 (k & 1) added per step
  // V transposing read: lane 16G + 4e + q addresses token 4(G >> 1) + e (and + 8),
  // column chunk 4(G & 1) + q of the fragment
  const int vG = lane >> 4, ve = (lane >> 2) & 3, vq = lane & 3;
  const int v_lo = v_chunk(4 * (vG >> 1) + ve, 4 * (vG & 1) + vq);
  const int v_hi = v_chunk(4 * (vG >> 1) + ve + 8, 4 * (vG & 1) + vq);

  // S^T of this wave's 32-token block of the tile staged at `kt`
  auto qk = [&](const lds_u8* kt, f32x16& S) {
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = 0.f;
    const lds_u8* kp = kt + (2 * ks + (r32 >> 4)) * KB * FRAG + k_pos;
#pragma unroll
    for (int k = 0; k < KS16; ++k) {
      const bf16x8 ka = *reinterpret_cast<lds_bf16x8*>(kp + (k >> 1) * FRAG + 512 * (k & 1));
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[k], S, 0, 0, 0);
    }
  };
  // causal mask of the block whose tile starts at t0 (only where it reaches past the first
  // row's limit)
  auto mask = [&](f32x16& S, int t0) {
    if constexpr (VAR) {
      if (var.k1 > 0.f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) S[i] = var.cap(S[i]);
      }
      if (var.masked || t0 + 32 * (ks + 1) > min_lim || t0 + 32 * ks < var.max_lo) {
        const uint32_t win = var.window(a.mask, t0 + 32 * ks);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int k = 8 * (i >> 2) + 4 * h + (i & 3), tok = t0 + 32 * ks + k;
          S[i] = var.keeps_at(win, k, tok, lim) ? S[i] : kNegInf;
        }
      }
    } else if (t0 + 32 * (ks + 1) > min_lim) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = t0 + 32 * ks + 8 * (i >> 2) + 4 * h + (i & 3);
        if (tok >= lim) S[i] = kNegInf;
      }
    }
  };
  // online softmax of one block's scores: update the reference m (raised only past the
  // margin; corr is this row's rescale factor, 1 when it stays) and l, write P as bf16 pairs;
  // returns whether any row of the wave raised its reference
  auto softmax = [&](const f32x16& S, uint32_t (&pk)[8]) -> bool {
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(S[i], S[i + 1]));
    const float mxs = pair_max(mx) * c;
    const bool raise = mxs > m + kRescaleMargin;
    const bool any = __ballot(raise) != 0;
    if (any) {
      const float mnew = raise ? mxs : m;
      corr = fast_exp2(m - mnew);  // 1 where the reference stays
      m = mnew;
      l *= corr;
    }
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(S[i], c, -m));
      const float p1 = fast_exp2(__builtin_fmaf(S[i + 1], c, -m));
      pk[i >> 1] = cvt_pk_bf16(p0, p1);
      lsum = sum_pair(pk[i >> 1], lsum);
    }
    l += lsum;
    return any;
  };
  auto rescale = [&](bool any) {
    if (any) {
#pragma unroll
      for (int b = 0; b < KB; ++b) oacc[b] *= corr;
    }
  };
  // O^T += V^T P^T over this wave's block of the tile staged at `vt`, one 16-token k-block
  // at a time
  auto pv = [&](const lds_u8* vt, const uint32_t (&pk)[8]) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const bf16x8 pb = __builtin_bit_cast(
          bf16x8, u32x4{pk[4 * half], pk[4 * half + 1], pk[4 * half + 2], pk[4 * half + 3]});
      const lds_u8* vf = vt + (2 * ks + half) * KB * FRAG;
#pragma unroll
      for (int cb = 0; cb < KB; ++cb) {
        const bf16x8 va = cat(tr_read(vf + cb * FRAG + v_lo), tr_read(vf + cb * FRAG + v_hi));
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[cb], 0, 0, 0);
      }
    }
  };

  if constexpr (!PIPE) {
    tile_loop<D>(pgn, item.kv_start, kv_end, sl, K, V, [&](const lds_u8* kt, const lds_u8* vt, int t0) {
      f32x16 S;
      uint32_t pk[8];
      qk(kt, S);
      mask(S, t0);
      rescale(softmax(S, pk));
      pv(vt, pk);
    });
  } else {
    // Software pipeline over 32-token tiles j (tokens T(j) .. T(j)+31); K(j) and V(j) sit in
    // slot j % 4 of their 4-slot rings (8 KB each for D = 128).  Step j, after one barrier:
    //   - DMA K(j+4) into K(j)'s slot and V(j+2) into V(j-2)'s slot (both read in step j-1);
    //   - one interleaved stream of matrix instructions: the scores of tile j+1
    //     (S(j+1) = K(j+1) Q^T, a chain of D/16 products) alternating with P.V of tile j-1
    //     (independent accumulators), while the vector ALUs run the online softmax of tile j
    //     (scores computed in step j-1) and produce P(j);
    //   - if the reference maximum was raised, rescale O (which now holds P.V up to j-1).
    // Every load is issued three steps before its use; each step issues one batch of D/64
    // loads of K and one of V per wave, so at the wait the batches younger than the ones
    // needed are those of the previous two steps (fewer where loads past the end were skipped).
    constexpr int NF = KB / 2;           // K (or V) fragments each wave loads per tile
    constexpr int HALF = 2 * KB * FRAG;  // bytes of K (or V) of one 32-token tile
    constexpr int AH = 2;                // operand reads issued ahead of their matrix instruction
    const int kv0 = item.kv_start;
    const int n = (kv_end - kv0 + 31) / 32;
    auto T = [&](int j) { return kv0 + 32 * j; };
    auto k_slot = [&](int j) { return sl.k0() + ((j >> 1) & 1) * PF<D>::SLOT + (j & 1) * HALF; };
    auto v_slot = [&](int j) { return sl.v0() + ((j >> 1) & 1) * PF<D>::SLOT + (j & 1) * HALF; };
    // wave w loads fragments w*NF .. w*NF+NF-1 (token group f / KB, column group f % KB)
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int f0 = wu * NF, tg = f0 / KB, cg = f0 % KB;
    auto page_k = [&](int j) { return pgn.page_of(T(j) + 16 * tg + k_dma_token(lane)); };
    auto page_v = [&](int j) { return pgn.page_of(T(j) + 16 * tg + v_dma_token(lane)); };
    auto dma_k = [&](int j, int32_t page) {
      dma_fragments<NF>(K + pgn.template row<D>(T(j) + 16 * tg + k_dma_token(lane), page) + 8 * (lane >> 4) + 32 * cg,
                        k_slot(j) + f0 * FRAG);
    };
    auto dma_v = [&](int j, int32_t page) {
      dma_fragments<NF>(V + pgn.template row<D>(T(j) + 16 * tg + v_dma_token(lane), page) + 8 * (lane >> 4) + 32 * cg,
                        v_slot(j) + f0 * FRAG);
    };
    // Fast steps (P divides 32) touch only full tiles (no clamping), and a lane's token keeps
    // its offset inside the page from tile to tile: its row address is the page id times the
    // page's bytes plus a per-item constant (one 32 x 32 -> 64-bit multiply-add), and its
    // page-table entry advances by 32 / P entries per tile.
    uint64_t k_add = 0, v_add = 0;
    int32_t k_pn = 0, v_pn = 0, pstep = 0;
    uint32_t page_bytes = 0;
    if constexpr (PG == kPageDiv32) {
      const int kx = kv0 + 16 * tg + k_dma_token(lane), vx = kv0 + 16 * tg + v_dma_token(lane);
      const int col = 8 * (lane >> 4) + 32 * cg;
      k_add = reinterpret_cast<uint64_t>(K) + 2u * uint32_t(((kx & (a.P - 1)) * a.Hk + hk) * D + col);
      v_add = reinterpret_cast<uint64_t>(V) + 2u * uint32_t(((vx & (a.P - 1)) * a.Hk + hk) * D + col);
      k_pn = kx >> a.p_shift;
      v_pn = vx >> a.p_shift;
      pstep = 32 >> a.p_shift;
      page_bytes = uint32_t(a.P * a.Hk * D) * 2u;
    }
    auto page_k_fast = [&](int j) { return pgn.table[k_pn + j * pstep - pgn.base]; };
    auto page_v_fast = [&](int j) { return pgn.table[v_pn + j * pstep - pgn.base]; };
    auto dma_k_fast = [&](int j, int32_t page) {
      const uint64_t addr = uint64_t(uint32_t(page)) * page_bytes + k_add;
      dma_fragments<NF>(reinterpret_cast<const uint16_t*>(addr), k_slot(j) + f0 * FRAG);
    };
    auto dma_v_fast = [&](int j, int32_t page) {
      const uint64_t addr = uint64_t(uint32_t(page)) * page_bytes + v_add;
      dma_fragments<NF>(reinterpret_cast<const uint16_t*>(addr), v_slot(j) + f0 * FRAG);
    };

    const float inv_c = 1.f / c;
    float thr = __builtin_fmaf(m, inv_c, kRescaleMargin * inv_c);  // raw-score threshold of a raise

    // One step's matrix and vector work in a fixed instruction order (scheduling barriers
    // between the groups keep the compiler from regrouping them): for g = 0 .. D/16 - 1,
    // P.V product g of tile j-1, score product g of tile j+1, the operand reads AH products
    // ahead, and slice g of the softmax of tile j (first the row maximum and the reference
    // update, then the exponentials, a few pairs per slice).  Returns whether any row of the
    // wave raised its reference (then corr holds each row's factor and l is already rescaled).
    auto fused = [&](const lds_u8* kt, const lds_u8* vt, f32x16& Snext, const f32x16& Scur, const u32x4 (&pprev)[2],
                     u32x4 (&pcur)[2]) -> bool {
      constexpr bool QK = true, PV = true, SM = true;
      const lds_u8* kp = kt + (r32 >> 4) * KB * FRAG + k_pos;
      auto kread = [&](int k) { return *reinterpret_cast<lds_bf16x8*>(kp + (k >> 1) * FRAG + 512 * (k & 1)); };
      // operand of P.V product m2 = (16-token half m2 / KB, column block m2 % KB)
      auto vread = [&](int m2) {
        const lds_u8* vf = vt + (m2 / KB) * KB * FRAG + (m2 % KB) * FRAG;
        return cat(tr_read(vf + v_lo), tr_read(vf + v_hi));
      };
      bf16x8 kr[KS16], va[KS16];
#pragma unroll
      for (int k = 0; k < AH; ++k) {
        if (PV) va[k] = vread(k);
        if (QK) kr[k] = kread(k);
      }
      float mx = 0.f, mx5[5], lsum = 0.f;
      bool any = false;
#pragma unroll
      for (int g = 0; g < KS16; ++g) {
        __builtin_amdgcn_sched_barrier(0);
        if (PV) {
          const int half = g / KB, cb = g % KB;
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[g], __builtin_bit_cast(bf16x8, pprev[half]), oacc[cb],
                                                             0, 0, 0);
        }
        if (QK) Snext = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[g], qb[g], g == 0 ? f32x16{} : Snext, 0, 0, 0);
        if (g + AH < KS16) {
          if (PV) va[g + AH] = vread(g + AH);
          if (QK) kr[g + AH] = kread(g + AH);
        }
        if (!SM) continue;
        if (g == 0) {
          // row maximum as a balanced tree of three-input maxima: five independent ones here
#pragma unroll
          for (int i = 0; i < 5; ++i) mx5[i] = fmaxf(Scur[3 * i], fmaxf(Scur[3 * i + 1], Scur[3 * i + 2]));
        } else if (g == 1) {
          mx = fmaxf(fmaxf(mx5[0], fmaxf(mx5[1], mx5[2])), fmaxf(mx5[3], fmaxf(mx5[4], Scur[15])));
          // the reference is raised when a raw score exceeds thr = (m + margin) / c
          const float pmx = pair_max(mx);
          const bool raise = pmx > thr;
          any = __ballot(raise) != 0;
          if (any) {  // rare after the first tiles: a scalar branch around the update
            const float mnew = raise ? pmx * c : m;
            corr = fast_exp2(m - mnew);  // 1 where the reference stays
            m = mnew;
            thr = __builtin_fmaf(m, inv_c, kRescaleMargin * inv_c);
            l *= corr;
          }
        } else {
          // pairs whose slice is g: pair q goes to slice 2 + q (KS16 - 2) / 8
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            if (2 + q * (KS16 - 2) / 8 != g) continue;
            const float p0 = fast_exp2(__builtin_fmaf(Scur[2 * q], c, -m));
            const float p1 = fast_exp2(__builtin_fmaf(Scur[2 * q + 1], c, -m));
            pcur[q >> 2][q & 3] = cvt_pk_bf16(p0, p1);
            lsum = sum_pair(pcur[q >> 2][q & 3], lsum);
          }
        }
      }
      // keep P and the scores inside this stream: without these the compiler sinks them next
      // to their first use, after the rescale branch
      pin(pcur);
      pin(Snext);
      asm volatile("" : "+v"(lsum));  // (the row sum too)
      __builtin_amdgcn_sched_barrier(0);
      l += lsum;
      return any;
    };

    f32x16 Sa, Sb;
    u32x4 pa[2], pb[2];
    __syncthreads();  // LDS free (previous item finished)
    pgn.base = -kPageWindow;  // nothing staged for this item yet
    pgn.template cover<kThreads, true>(T(0), T(kKAhead + 2) - 1);
    const bool window_holds_item = pgn.page_no(kv_end - 1) - pgn.base < kPageWindow;  // (uniform)
    {
      int32_t kp[kKAhead], vp[kVAhead];
#pragma unroll
      for (int i = 0; i < kKAhead; ++i) kp[i] = page_k(i);
#pragma unroll
      for (int i = 0; i < kVAhead; ++i) vp[i] = page_v(i);
#pragma unroll
      for (int i = 0; i < kKAhead; ++i)
        if (i == 0 || n > i) dma_k(i, kp[i]);
#pragma unroll
      for (int i = 0; i < kVAhead; ++i)
        if (i == 0 || n > i) dma_v(i, vp[i]);
    }
    int32_t nk = page_k(kKAhead), nv = page_v(kVAhead);  // for step 0's loads
    BSR_WAIT_VMCNT(0);
    __syncthreads();  // K(0 .. kKAhead-1), V(0 .. kVAhead-1) staged
    qk(k_slot(0), Sa);
    mask(Sa, T(0));

    // Steps 0 .. n all run the same stream.  In step 0 the P.V product uses P(-1) = 0 over
    // the staged V(0) (rows of real tokens, so it adds exact zeros).  Step n-1 computes the
    // scores of the nonexistent tile n from a stale slot and the mask sets every one of them
    // to -inf (all its tokens lie past the end), so step n's softmax leaves the state as it
    // is while its P.V product adds the last tile.
    // Fast steps need tiles up to j + 5 full (and exist only for P dividing 32).
    const int n_full = PG == kPageDiv32 ? (kv_end - kv0) / 32 : 0;
    // step j with S(j) in Scur and P(j-1) in pprev; writes S(j+1) to Snext and P(j) to pcur
    auto step = [&](int j, f32x16& Scur, f32x16& Snext, const u32x4 (&pprev)[2], u32x4 (&pcur)[2]) {
      const bool fast = PG == kPageDiv32 && j >= 1 && j + kKAhead + 1 < n_full;
      // this step's lookups: K(j + kKAhead + 1), V(j + kVAhead + 1) (the window filled at the
      // item's start holds all of its pages unless the item spans more than kPageWindow)
      if (!window_holds_item) pgn.cover(T(j + kVAhead + 1), T(j + kKAhead + 2) - 1);
      wait_dma_batches<NF>(fast ? kMaxBatchesInFlight : batches_in_between(j, n));
      __builtin_amdgcn_s_barrier();
      if (fast) {
        const int32_t nk2 = page_k_fast(j + kKAhead + 1), nv2 = page_v_fast(j + kVAhead + 1);
        dma_k_fast(j + kKAhead, nk);
        dma_v_fast(j + kVAhead, nv);
        nk = nk2;
        nv = nv2;
      } else {
        const int32_t nk2 = page_k(j + kKAhead + 1), nv2 = page_v(j + kVAhead + 1);
        if (j + kKAhead < n) dma_k(j + kKAhead, nk);
        if (j + kVAhead < n) dma_v(j + kVAhead, nv);
        nk = nk2;
        nv = nv2;
      }
      __builtin_amdgcn_sched_barrier(0);
      const bool any = fused(k_slot(j + 1), v_slot(j == 0 ? 0 : j - 1), Snext, Scur, pprev, pcur);
      rescale(any);
      mask(Snext, T(j + 1));
    };
    // Steady steps, as in the 128-row shape: the steps j (from a multiple of 4 on) for which the
    // window holds the item, the lookahead tiles are full tiles of the fast page class, the wait
    // is for kMaxBatchesInFlight batches and (without VAR) the next score tile needs no mask run
    // as straight-line code, four per loop trip, with every LDS slot known at compile time.  With
    // VAR the mask (which also applies the soft cap and the custom mask) runs in every step.
    int j_fast = -1, n_quads = 0;  // (uniform)
    if constexpr (PG == kPageDiv32) {
      if (window_holds_item) {
        int hi = n_full - kKAhead - 2;                                    // j + kKAhead + 1 < n_full
        if constexpr (!VAR) hi = min(hi, (min_lim - kv0) / 32 - 2);       // T(j + 1) + 32 <= min_lim
        constexpr int lo = 4;                                             // (V(j - 1) exists from j = 1)
        if (hi >= lo) {
          j_fast = lo;
          n_quads = (hi - lo + 1) / 4;
        }
      }
    }
    const uint32_t lds_k = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sl.k0() + f0 * FRAG)));
    const uint32_t lds_v = __builtin_amdgcn_readfirstlane(
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sl.v0() + f0 * FRAG)));
    auto slot_off = [](int j) { return ((j >> 1) & 1) * PF<D>::SLOT + (j & 1) * HALF; };
    auto fast_step = [&](auto qc, int j, f32x16& Scur, f32x16& Snext, const u32x4 (&pprev)[2], u32x4 (&pcur)[2]) {
      constexpr int q = decltype(qc)::value;  // j mod 4
      BSR_WAIT_VMCNT(kMaxBatchesInFlight * NF);
      __builtin_amdgcn_s_barrier();
      const int32_t nk2 = page_k_fast(j + kKAhead + 1), nv2 = page_v_fast(j + kVAhead + 1);
      dma_kv<NF>(reinterpret_cast<const uint16_t*>(uint64_t(uint32_t(nk)) * page_bytes + k_add),
                 lds_k + slot_off((q + kKAhead) & 3),
                 reinterpret_cast<const uint16_t*>(uint64_t(uint32_t(nv)) * page_bytes + v_add),
                 lds_v + slot_off((q + kVAhead) & 3));
      nk = nk2;
      nv = nv2;
      __builtin_amdgcn_sched_barrier(0);
      const bool any = fused(sl.k0() + slot_off((q + 1) & 3), sl.v0() + slot_off((q + 3) & 3), Snext, Scur, pprev, pcur);
      rescale(any);
      if constexpr (VAR) mask(Snext, T(j + 1));
    };
    using Q0 = std::integral_constant<int, 0>;
    using Q1 = std::integral_constant<int, 1>;
    using Q2 = std::integral_constant<int, 2>;
    using Q3 = std::integral_constant<int, 3>;
#pragma unroll
    for (int i = 0; i < 2; ++i) pb[i] = u32x4{0u, 0u, 0u, 0u};  // P(-1)
    // two steps per iteration so that the register roles alternate without copies
    for (int j = 0;; j += 2) {
      if (j == j_fast) {
        for (int i = 0; i < n_quads; ++i, j += 4) {
          fast_step(Q0{}, j, Sa, Sb, pb, pa);
          fast_step(Q1{}, j + 1, Sb, Sa, pa, pb);
          fast_step(Q2{}, j + 2, Sa, Sb, pb, pa);
          fast_step(Q3{}, j + 3, Sb, Sa, pa, pb);
        }
      }
      step(j, Sa, Sb, pb, pa);
      if (j + 1 > n) break;
      step(j + 1, Sb, Sa, pa, pb);
      if (j + 2 > n) break;
    }
  }

  l = pair_sum(l);  // the two halves of a row held different tokens

  if constexpr (N_KS > 1) {
    // combine the two waves that split each row block's tokens: the second one publishes
    // its state, the first one folds it in (the loop ended with a barrier: LDS is free)
    lds_f32* comb = reinterpret_cast<lds_f32*>(rg == 0 ? sl.v0() : sl.v1());
    if (ks == 1 && rb_on) {
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) comb[r32 * (D + 2) + 32 * b + 8 * (i >> 2) + 4 * h + (i & 3)] = oacc[b][i];
      if (h == 0) {
        comb[r32 * (D + 2) + D] = m;
        comb[r32 * (D + 2) + D + 1] = l;
      }
    }
    __syncthreads();
    if (ks == 0 && rb_on) {
      const float m2 = comb[r32 * (D + 2) + D], l2 = comb[r32 * (D + 2) + D + 1];
      const float mm = fmaxf(m, m2);
      const float muse = mm == kNegInf ? 0.f : mm;
      const float w1 = fast_exp2(m - muse), w2 = fast_exp2(m2 - muse);
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          oacc[b][i] = w1 * oacc[b][i] + w2 * comb[r32 * (D + 2) + 32 * b + 8 * (i >> 2) + 4 * h + (i & 3)];
      l = w1 * l + w2 * l2;
      m = mm;
    }
  }

  // ---- epilogue: final output or partial state ----
  if (ks == 0 && row_ok) {
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    const float lse = empty ? kNegInf : (m + log2f(l)) * kLn2;
    if (item.slot < 0) {
      const int64_t orow = int64_t(rq.q_start + row_pos) * a.Hq + row_hq;
      uint16_t* op = static_cast<uint16_t*>(a.o) + orow * D + 4 * h;
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<u32x2*>(op + 32 * b + 8 * q4) =
              u32x2{cvt_pk_bf16(oacc[b][4 * q4] * inv, oacc[b][4 * q4 + 1] * inv),
                    cvt_pk_bf16(oacc[b][4 * q4 + 2] * inv, oacc[b][4 * q4 + 3] * inv)};
      if (h == 0) a.lse[orow] = lse;
    } else {
      const int64_t prow = (int64_t(item.slot) * a.Hk + hk) * a.Tq + (r - item.row_start);
      float* pp = a.part_o + prow * D + 4 * h;
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(pp + 32 * b + 8 * q4) =
              f32x4{oacc[b][4 * q4], oacc[b][4 * q4 + 1], oacc[b][4 * q4 + 2], oacc[b][4 * q4 + 3]} * inv;
      if (h == 0) a.part_lse[prow] = lse;
    }
  }
}

// ---------------------------------------------------------------------------------
// Small query tiles (<= 32 rows): 16-row blocks on v_mfma_f32_16x16x32_bf16.
// NT: 16-token blocks of a tile per wave (2: two waves per row block, 1: four).
// ---------------------------------------------------------------------------------
template <int D, int NT, bool POW2, bool VAR>
__device__ __forceinline__ void prefill_item16(const RunArgs& a, const ItemRec& item, const ReqRec& rq, int hk,
                                               const Slots<D>& sl) {
  constexpr int KB = PF<D>::KB, DB = D / 16, FRAG = PF<D>::FRAG;
  constexpr int N_KS = 4 / NT;  // waves sharing a row block
  constexpr int N_RG = kWaves / N_KS;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, j = lane >> 4;
  const int rg = wave % N_RG, ks = wave / N_RG;
  const int nrows = item.row_end - item.row_start;
  const float c = a.sm_scale * kLog2e;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  const int kv_end = item.kv_end;
  Paging<POW2> pgn{a.indices, sl.table(), rq.page_start, a.P, a.p_shift, a.Hk, hk, kv_end, -kPageWindow};

  const int r = item.row_start + rg * 16 + n;
  const bool rb_on = rg * 16 < nrows;
  const bool row_ok = r < item.row_end;
  const int row_pos = r / a.g, row_hq = hk * a.g + r % a.g;
  const int lim = (a.causal && row_ok) ? min(kv_end, rq.kv_len - rq.q_len + row_pos + 1) : kv_end;
  const VarRow var(a, item, rq, row_pos, row_ok);
  bf16x8 qb[KB];
  {
    const uint16_t* qp = Q + (int64_t(rq.q_start + row_pos) * a.Hq + row_hq) * D + j * 8;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4*>(qp + kb * 32);
      qb[kb] = __builtin_bit_cast(bf16x8, v);
    }
  }
  int min_lim = kv_end;
  if (a.causal) min_lim = min(kv_end, rq.kv_len - rq.q_len + item.row_start / a.g + 1);

  float m = kNegInf, l = 0.f;
  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // V transposing read: lane 16G + 4e + q addresses token 4G + e, column chunk q of the
  // 16-wide block (chunk 4(db & 1) + q of the fragment)
  const int vG = lane >> 4, ve = (lane >> 2) & 3, vq = lane & 3;
  const int v_even = v_chunk(4 * vG + ve, vq), v_odd = v_chunk(4 * vG + ve, 4 + vq);

  auto compute = [&](const lds_u8* kt, const lds_u8* vt, int t0) {
    f32x4 S[NT];
#pragma unroll
    for (int b = 0; b < NT; ++b) S[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const int tb = ks * NT + b;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 ka = *reinterpret_cast<lds_bf16x8*>(kt + (tb * KB + kb) * FRAG + lane * 16);
        S[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[kb], S[b], 0, 0, 0);
      }
    }
    if constexpr (VAR) {
      if (var.k1 > 0.f) {
#pragma unroll
        for (int b = 0; b < NT; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[b][i] = var.cap(S[b][i]);
      }
      if (var.masked || t0 + kTileKV > min_lim || t0 < var.max_lo) {
        const int tb = t0 + ks * NT * 16;  // this wave's keys: tb .. tb + 16 NT - 1 (NT <= 2)
        const uint32_t win = var.window(a.mask, tb);
#pragma unroll
        for (int b = 0; b < NT; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = b * 16 + 4 * j + i, tok = tb + k;
            S[b][i] = var.keeps_at(win, k, tok, lim) ? S[b][i] : kNegInf;
          }
      }
    } else if (t0 + kTileKV > min_lim) {
#pragma unroll
      for (int b = 0; b < NT; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = t0 + (ks * NT + b) * 16 + 4 * j + i;
          if (tok >= lim) S[b][i] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int b = 0; b < NT; ++b) mx = fmaxf(fmaxf(mx, fmaxf(S[b][0], S[b][1])), fmaxf(S[b][2], S[b][3]));
    mx = pair16_max(mx);
    mx = pair_max(mx);
    bool any;
    const float corr = raise_reference(m, mx * c, any);
    if (any) {
      l *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= corr;
    }
    const float muse = m == kNegInf ? 0.f : m;
    uint32_t pk[NT][2];
    float lsum = 0.f;
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(__builtin_fmaf(S[b][i], c, -muse));
      pk[b][0] = cvt_pk_bf16(p[0], p[1]);
      pk[b][1] = cvt_pk_bf16(p[2], p[3]);
      lsum = sum_pair(pk[b][1], sum_pair(pk[b][0], lsum));
    }
    l += lsum;
    if constexpr (NT >= 2) {
#pragma unroll
      for (int b = 0; b < NT; b += 2) {
        const int tba = ks * NT + b, tbb = tba + 1;
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[b][0], pk[b][1], pk[b + 1][0], pk[b + 1][1]});
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int off = (db >> 1) * FRAG + ((db & 1) ? v_odd : v_even);
          const bf16x8 vab = cat(tr_read(vt + tba * KB * FRAG + off), tr_read(vt + tbb * KB * FRAG + off));
          oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vab, pb, oacc[db], 0, 0, 0);
        }
      }
    } else {
      const int tb = ks;
      const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{pk[0][0], pk[0][1]});
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int off = (db >> 1) * FRAG + ((db & 1) ? v_odd : v_even);
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(tr_read(vt + tb * KB * FRAG + off), pb, oacc[db], 0, 0, 0);
      }
    }
  };
  tile_loop<D>(pgn, item.kv_start, kv_end, sl, K, V, compute);

  l = pair16_sum(l);
  l = pair_sum(l);

  {
    // combine the waves that split this row block's tokens; waves 0-1 use the first
    // stage's array, waves 2-3 the second one's
    auto comb_of = [&](int wv) -> lds_f32* {
      return reinterpret_cast<lds_f32*>((wv < 2 ? sl.v0() : sl.v1()) + (wv & 1) * PF<D>::COMB16);
    };
    lds_f32* mine = comb_of(wave);
    if (rb_on) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[n * (D + 2) + db * 16 + 4 * j + i] = oacc[db][i];
      if (j == 0) {
        mine[n * (D + 2) + D] = m;
        mine[n * (D + 2) + D + 1] = l;
      }
    }
    __syncthreads();
    if (ks == 0 && rb_on) {
      float mm = kNegInf;
#pragma unroll
      for (int o = 0; o < N_KS; ++o) mm = fmaxf(mm, comb_of(rg + o * N_RG)[n * (D + 2) + D]);
      const float muse = mm == kNegInf ? 0.f : mm;
      float lt = 0.f, wgt[N_KS];
#pragma unroll
      for (int o = 0; o < N_KS; ++o) {
        const lds_f32* src = comb_of(rg + o * N_RG) + n * (D + 2);
        wgt[o] = fast_exp2(src[D] - muse);
        lt += wgt[o] * src[D + 1];
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sum = 0.f;
#pragma unroll
          for (int o = 0; o < N_KS; ++o) sum += wgt[o] * comb_of(rg + o * N_RG)[n * (D + 2) + db * 16 + 4 * j + i];
          oacc[db][i] = sum;
        }
      m = mm;
      l = lt;
    }
  }

  if (ks == 0 && row_ok) {
    const bool empty = !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    const float lse = empty ? kNegInf : (m + log2f(l)) * kLn2;
    if (item.slot < 0) {
      const int64_t orow = int64_t(rq.q_start + row_pos) * a.Hq + row_hq;
      uint16_t* op = static_cast<uint16_t*>(a.o) + orow * D + 4 * j;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4 v = oacc[db] * inv;
        *reinterpret_cast<u32x2*>(op + db * 16) = u32x2{cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3])};
      }
      if (j == 0) a.lse[orow] = lse;
    } else {
      const int64_t prow = (int64_t(item.slot) * a.Hk + hk) * a.Tq + (r - item.row_start);
      float* pp = a.part_o + prow * D + 4 * j;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(pp + db * 16) = oacc[db] * inv;
      if (j == 0) a.part_lse[prow] = lse;
    }
  }
}

// ---------------------------------------------------------------------------------
// Query tiles of up to 128 rows on two waves of 512 VGPRs (one wave per SIMD, two
// workgroups per CU).  Wave w holds row blocks 2w and 2w+1 (32 rows each), so every K
// fragment and every V operand read from LDS feeds two matrix instructions, and each
// staged 32-token KV tile serves all 128 rows.  The step structure is the software
// pipeline of the 4-wave shape: after one barrier per step, the scores of tile j+1
// (S(j+1) = K(j+1) Q^T) and P.V of tile j-1 run on the matrix cores while the vector ALUs
// run the online softmax of tile j, for both row blocks.  Absent rows (past the end of a
// short tile) carry zero queries and are never written.
// ---------------------------------------------------------------------------------
template <int D, int PG, bool VAR>
__device__ __forceinline__ void prefill_item128(const RunArgs& a, const ItemRec& item, const ReqRec& rq, int hk,
                                                const Slots<D>& sl, const RecFetch& nf) {
  constexpr int KB = PF<D>::KB, FRAG = PF<D>::FRAG;
  constexpr int KS16 = D / 16;  // 16-deep k-steps of the score product
  constexpr bool POW2 = PG != kPageAny;
  constexpr int NF = KB;               // fragments of K (or V) each wave loads per tile
  constexpr int HALF = 2 * KB * FRAG;  // bytes of K (or V) of one 32-token tile
  constexpr int AH = 2;                // operand reads issued ahead of their matrix instructions
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r32 = lane & 31, h = lane >> 5;
  const float c = a.sm_scale * kLog2e;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  const int kv_end = item.kv_end;
  Paging<POW2> pgn{a.indices, sl.table(), rq.page_start, a.P, a.p_shift, a.Hk, hk, kv_end, -kPageWindow};

  // this lane's query rows: row r32 of blocks 2 wave and 2 wave + 1
  int row_pos[2], row_hq[2], lim[2];
  bool row_ok[2];
  bf16x8 qb[2][KS16];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int r = item.row_start + 64 * wave + 32 * b + r32;
    row_ok[b] = r < item.row_end;
    row_pos[b] = r / a.g;
    row_hq[b] = hk * a.g + r % a.g;
    lim[b] = (a.causal && row_ok[b]) ? min(kv_end, rq.kv_len - rq.q_len + row_pos[b] + 1) : kv_end;
    const uint16_t* qp = Q + (int64_t(rq.q_start + row_pos[b]) * a.Hq + row_hq[b]) * D + 8 * h;
#pragma unroll
    for (int k = 0; k < KS16; ++k) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok[b]) v = *reinterpret_cast<const u32x4*>(qp + 16 * k);
      qb[b][k] = __builtin_bit_cast(bf16x8, v);
    }
  }
  int min_lim = kv_end;  // tiles ending before the smallest visible end need no mask
  if (a.causal) min_lim = min(kv_end, rq.kv_len - rq.q_len + item.row_start / a.g + 1);
  min_lim = __builtin_amdgcn_readfirstlane(min_lim);
  const VarRow var[2] = {VarRow(a, item, rq, row_pos[0], row_ok[0]), VarRow(a, item, rq, row_pos[1], row_ok[1])};

  // running references (log2 units, from a finite floor), sums and rescale factors per block
  float m[2] = {kMFloor, kMFloor}, l[2] = {0.f, 0.f}, corr[2] = {1.f, 1.f};
  const float inv_c = 1.f / c;
  float thr[2];  // raw-score threshold of a raise: (m + margin) / c
#pragma unroll
  for (int b = 0; b < 2; ++b) thr[b] = __builtin_fmaf(m[b], inv_c, kRescaleMargin * inv_c);
  f32x16 oacc[2][KB];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int cb = 0; cb < KB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[b][cb][i] = 0.f;

  // LDS layout of this shape: in a 1 KB fragment (16 tokens x 32 columns) the four 16-byte
  // chunks of token t fill slots 4t .. 4t+3, so that each lane quad of an LDS-DMA load reads
  // one token's 64 contiguous bytes (four quads on four rows cost about a quarter of sixteen
  // lanes on sixteen rows in the texture path); K chunk c of token t sits at slot
  // 4t + (c ^ ((t >> 2) & 3)), which puts the 16 tokens of one chunk read in 16 different bank
  // groups; V is not swizzled (a transposing read spans four tokens 64 bytes apart).
  // K read of k-step k by lane (token r32, half h): chunk 2 (k & 1) + h of token r32 & 15.
  const int kt16 = r32 & 15, ksw = (kt16 >> 2) & 3;
  const int k_pos0 = 16 * (4 * kt16 + (h ^ ksw)), k_pos1 = 16 * (4 * kt16 + ((2 + h) ^ ksw));
  // V transposing read: lane 16G + 4e + q addresses token 4(G >> 1) + e (and + 8), 8-byte
  // column unit 4(G & 1) + q
  const int vG = lane >> 4, ve = (lane >> 2) & 3, vq = lane & 3;
  const int v_lo = 64 * (4 * (vG >> 1) + ve) + 8 * (4 * (vG & 1) + vq);
  const int v_hi = v_lo + 512;
  // DMA lane roles: token lane >> 2 of the wave's 16, chunk (K swizzled as above)
  const int d_tok = lane >> 2, dk_col = 8 * ((lane & 3) ^ ((lane >> 4) & 3)), dv_col = 8 * (lane & 3);

  const int kv0 = item.kv_start;
  const int n = (kv_end - kv0 + 31) / 32;
  auto T = [&](int j) { return kv0 + 32 * j; };
  auto k_slot = [&](int j) { return sl.k0() + ((j >> 1) & 1) * PF<D>::SLOT + (j & 1) * HALF; };
  auto v_slot = [&](int j) { return sl.v0() + ((j >> 1) & 1) * PF<D>::SLOT + (j & 1) * HALF; };

  // scores of both blocks for the tile staged at `kt` (prologue only)
  auto qk = [&](const lds_u8* kt, f32x16 (&S)[2]) {
    const lds_u8* kp = kt + (r32 >> 4) * KB * FRAG;
#pragma unroll
    for (int k = 0; k < KS16; ++k) {
      const bf16x8 ka = *reinterpret_cast<lds_bf16x8*>(kp + (k >> 1) * FRAG + ((k & 1) ? k_pos1 : k_pos0));
#pragma unroll
      for (int b = 0; b < 2; ++b)
        S[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[b][k], k == 0 ? f32x16{} : S[b], 0, 0, 0);
    }
  };
  // causal mask of the tile starting at t0 (only where it reaches past the first row's limit)
  // (with VAR also below the sliding window's first key; soft-capped and custom-masked runs
  // never come here)
  auto mask = [&](f32x16 (&S)[2], int t0) {
    if constexpr (VAR) {
      if (t0 + 32 > min_lim || t0 < var[0].max_lo) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int tok = t0 + 8 * (i >> 2) + 4 * h + (i & 3);
            if (tok >= lim[b] || tok < var[b].lo) S[b][i] = kNegInf;
          }
      }
    } else if (t0 + 32 > min_lim) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = t0 + 8 * (i >> 2) + 4 * h + (i & 3);
          if (tok >= lim[b]) S[b][i] = kNegInf;
        }
    }
  };

  // wave w loads token group w (16 tokens) of every 32-token tile, all KB column groups
  auto page_k = [&](int j) { return pgn.page_of(T(j) + 16 * wave + d_tok); };
  auto page_v = page_k;  // K and V lanes carry the same tokens
  auto dma_k = [&](int j, int32_t page) {
    dma_fragments<NF>(K + pgn.template row<D>(T(j) + 16 * wave + d_tok, page) + dk_col, k_slot(j) + wave * KB * FRAG);
  };
  auto dma_v = [&](int j, int32_t page) {
    dma_fragments<NF>(V + pgn.template row<D>(T(j) + 16 * wave + d_tok, page) + dv_col, v_slot(j) + wave * KB * FRAG);
  };
  // fast steps (P divides 32): fixed in-page offsets, page-table entries advance by 32 / P
  uint64_t k_add = 0, v_add = 0;
  int32_t k_pn = 0, v_pn = 0, pstep = 0;
  uint32_t page_bytes = 0;
  if constexpr (PG == kPageDiv32) {
    const int kx = kv0 + 16 * wave + d_tok, vx = kx;
    k_add = reinterpret_cast<uint64_t>(K) + 2u * uint32_t(((kx & (a.P - 1)) * a.Hk + hk) * D + dk_col);
    v_add = reinterpret_cast<uint64_t>(V) + 2u * uint32_t(((vx & (a.P - 1)) * a.Hk + hk) * D + dv_col);
    k_pn = kx >> a.p_shift;
    v_pn = vx >> a.p_shift;
    pstep = 32 >> a.p_shift;
    page_bytes = uint32_t(a.P * a.Hk * D) * 2u;
  }
  auto page_k_fast = [&](int j) { return pgn.table[k_pn + j * pstep - pgn.base]; };
  auto page_v_fast = [&](int j) { return pgn.table[v_pn + j * pstep - pgn.base]; };
  auto dma_k_fast = [&](int j, int32_t page) {
    const uint64_t addr = uint64_t(uint32_t(page)) * page_bytes + k_add;
    dma_fragments<NF>(reinterpret_cast<const uint16_t*>(addr), k_slot(j) + wave * KB * FRAG);
  };
  auto dma_v_fast = [&](int j, int32_t page) {
    const uint64_t addr = uint64_t(uint32_t(page)) * page_bytes + v_add;
    dma_fragments<NF>(reinterpret_cast<const uint16_t*>(addr), v_slot(j) + wave * KB * FRAG);
  };

  // One step's stream: 4 D/16 slots s = 4g + m, each one matrix instruction followed by one
  // chunk of vector work, in a fixed order (scheduling barriers between the slots keep the
  // compiler from regrouping them; a single wave per SIMD issues in order, so a matrix
  // instruction is followed by about as much vector work as it takes to execute).
  //   m = 0, 1: P.V product g of block m (V operand g of tile j-1, P(j-1) of block m);
  //   m = 2, 3: score product g of block m - 2 (K fragment g of tile j+1).
  // Vector chunks (softmax of tile j): slots 0, 1 the leaves of each block's maximum tree,
  // 4, 5 the rest of the tree and the cross-lane maximum, 6 the reference update of both
  // blocks (selects, no branch), then 16 units of two exponentials (pair q of block b) spread
  // over slots 7 .. 4 D/16 - 1.  Operand reads are issued AH k-steps ahead.
  auto fused = [&](const lds_u8* kt, const lds_u8* vt, f32x16 (&Snext)[2], const f32x16 (&Scur)[2],
                   const u32x4 (&pprev)[2][2], u32x4 (&pcur)[2][2]) -> bool {
    constexpr int NS = 4 * KS16;
    const lds_u8* kp = kt + (r32 >> 4) * KB * FRAG;
    auto kread = [&](int k) {
      return *reinterpret_cast<lds_bf16x8*>(kp + (k >> 1) * FRAG + ((k & 1) ? k_pos1 : k_pos0));
    };
    auto vread = [&](int m2) {
      const lds_u8* vf = vt + (m2 / KB) * KB * FRAG + (m2 % KB) * FRAG;
      return cat(tr_read(vf + v_lo), tr_read(vf + v_hi));
    };
    bf16x8 kr[KS16], va[KS16];
#pragma unroll
    for (int k = 0; k < AH; ++k) {
      va[k] = vread(k);
      kr[k] = kread(k);
    }
    float mx5[2][5], pmx[2], lsum[2] = {0.f, 0.f};
    bool raise[2] = {false, false}, any = false;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int g = s >> 2, mm = s & 3;
      __builtin_amdgcn_sched_barrier(0);
      if (mm == 0 && g + AH < KS16) {  // operands of k-step g + AH
        va[g + AH] = vread(g + AH);
        kr[g + AH] = kread(g + AH);
      }
      if (mm < 2) {
        mfma_acc_agpr(oacc[mm][g % KB], va[g], __builtin_bit_cast(bf16x8, pprev[mm][g / KB]));
      } else {
        const int b = mm - 2;
        Snext[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[g], qb[b][g], g == 0 ? f32x16{} : Snext[b], 0, 0, 0);
      }
      if (s < 2) {
        // leaves of block s's maximum tree: five independent three-input maxima
#pragma unroll
        for (int i = 0; i < 5; ++i)
          mx5[s][i] = fmaxf(Scur[s][3 * i], fmaxf(Scur[s][3 * i + 1], Scur[s][3 * i + 2]));
      } else if (s == 4 || s == 5) {
        const int b = s - 4;
        const float mx = fmaxf(fmaxf(mx5[b][0], fmaxf(mx5[b][1], mx5[b][2])),
                               fmaxf(mx5[b][3], fmaxf(mx5[b][4], Scur[b][15])));
        pmx[b] = pair_max(mx);
        raise[b] = pmx[b] > thr[b];
      } else if (s == 6) {
        // the reference moves only where a raw score passed (m + margin) / c
        any = __ballot(raise[0] || raise[1]) != 0;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const float mnew = raise[b] ? pmx[b] * c : m[b];
          corr[b] = fast_exp2(m[b] - mnew);  // 1 where the reference stays
          m[b] = mnew;
          thr[b] = __builtin_fmaf(m[b], inv_c, kRescaleMargin * inv_c);
          l[b] *= corr[b];
        }
      } else if (s >= 7) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (7 + u * (NS - 7) / 16 != s) continue;
          const int b = u & 1, q = u >> 1;
          const float p0 = fast_exp2(__builtin_fmaf(Scur[b][2 * q], c, -m[b]));
          const float p1 = fast_exp2(__builtin_fmaf(Scur[b][2 * q + 1], c, -m[b]));
          pcur[b][q >> 2][q & 3] = cvt_pk_bf16(p0, p1);
          lsum[b] = sum_pair(pcur[b][q >> 2][q & 3], lsum[b]);
        }
      }
    }
    // keep P and the scores inside this stream: without these the compiler sinks them next
    // to their first use
    pin(pcur[0]);
    pin(pcur[1]);
    pin(Snext[0]);
    pin(Snext[1]);
    asm volatile("" : "+v"(lsum[0]), "+v"(lsum[1]));  // (the row sums too)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < 2; ++b) l[b] += lsum[b];
    return any;
  };
  auto rescale = [&](bool any) {
    if (any) {
      acc_settle();
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int cb = 0; cb < KB; ++cb) oacc[b][cb] *= corr[b];
      acc_settle();
    }
  };

  f32x16 Sa[2], Sb[2];
  u32x4 pa[2][2], pb[2][2];
  __syncthreads();  // LDS free (previous item finished)
  pgn.template cover<kThreads2, true>(T(0), T(kKAhead + 2) - 1);
  const bool window_holds_item = pgn.page_no(kv_end - 1) - pgn.base < kPageWindow;  // (uniform)
  {
    int32_t kp[kKAhead], vp[kVAhead];
#pragma unroll
    for (int i = 0; i < kKAhead; ++i) kp[i] = page_k(i);
#pragma unroll
    for (int i = 0; i < kVAhead; ++i) vp[i] = page_v(i);
#pragma unroll
    for (int i = 0; i < kKAhead; ++i)
      if (i == 0 || n > i) dma_k(i, kp[i]);
#pragma unroll
    for (int i = 0; i < kVAhead; ++i)
      if (i == 0 || n > i) dma_v(i, vp[i]);
  }
  int32_t nk = page_k(kKAhead), nv = page_v(kVAhead);  // for step 0's loads
  BSR_WAIT_VMCNT(0);
  nf.store(sl.rec());  // (its load was issued before this item's)
  __syncthreads();  // K(0 .. kKAhead-1), V(0 .. kVAhead-1) staged
  qk(k_slot(0), Sa);
  mask(Sa, T(0));

  // Steps 0 .. n as in prefill_item32: step 0's P.V uses P(-1) = 0 over V(0); the scores of
  // the nonexistent tile n are all masked, so step n only adds P.V of the last tile.
  const int n_full = PG == kPageDiv32 ? (kv_end - kv0) / 32 : 0;
  auto step = [&](int j, f32x16 (&Scur)[2], f32x16 (&Snext)[2], const u32x4 (&pprev)[2][2], u32x4 (&pcur)[2][2]) {
    const bool fast = PG == kPageDiv32 && j >= 1 && j + kKAhead + 1 < n_full;
    // lookups: K(j + kKAhead + 1), V(j + kVAhead + 1); the window filled at the item's start holds
    // all of its pages unless the item spans more than kPageWindow of them
    if (!window_holds_item) pgn.template cover<kThreads2>(T(j + kVAhead + 1), T(j + kKAhead + 2) - 1);
    wait_dma_batches<NF>(fast ? kMaxBatchesInFlight : batches_in_between(j, n));
    __builtin_amdgcn_s_barrier();
    if (fast) {
      const int32_t nk2 = page_k_fast(j + kKAhead + 1), nv2 = page_v_fast(j + kVAhead + 1);
      dma_k_fast(j + kKAhead, nk);
      dma_v_fast(j + kVAhead, nv);
      nk = nk2;
      nv = nv2;
    } else {
      const int32_t nk2 = page_k(j + kKAhead + 1), nv2 = page_v(j + kVAhead + 1);
      if (j + kKAhead < n) dma_k(j + kKAhead, nk);
      if (j + kVAhead < n) dma_v(j + kVAhead, nv);
      nk = nk2;
      nv = nv2;
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool any = fused(k_slot(j + 1), v_slot(j == 0 ? 0 : j - 1), Snext, Scur, pprev, pcur);
    rescale(any);
    mask(Snext, T(j + 1));
  };
  // Steady steps: the steps j (from a multiple of 4 on) for which every test of step() comes out
  // the same way: no window refill (the window holds the item), a full lookahead tile in the fast
  // page class, a wait for kMaxBatchesInFlight batches, and a next score tile that needs no mask.
  // They run as straight-line code, four per loop trip, so that j mod 4 and with it every LDS slot
  // is known at compile time; loads, waits and barriers are those step() would issue.
  int j_fast = -1, n_quads = 0;  // (uniform)
  if constexpr (PG == kPageDiv32) {
    if (window_holds_item) {
      int hi = n_full - kKAhead - 2;                // j + kKAhead + 1 < n_full
      hi = min(hi, (min_lim - kv0) / 32 - 2);       // T(j + 1) + 32 <= min_lim
      int lo = 1;                                   // V(j - 1) exists
      if constexpr (VAR) {
        if (var[0].max_lo > kv0) lo = max(lo, (var[0].max_lo - kv0 + 31) / 32 - 1);  // T(j + 1) >= max_lo
      }
      lo = (lo + 3) & ~3;
      if (hi >= lo) {
        j_fast = lo;
        n_quads = (hi - lo + 1) / 4;
      }
    }
  }
  const uint32_t lds_k = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sl.k0() + wave * KB * FRAG)));
  const uint32_t lds_v = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(sl.v0() + wave * KB * FRAG)));
  auto slot_off = [](int j) { return ((j >> 1) & 1) * PF<D>::SLOT + (j & 1) * HALF; };
  auto fast_step = [&](auto qc, int j, f32x16 (&Scur)[2], f32x16 (&Snext)[2], const u32x4 (&pprev)[2][2],
                       u32x4 (&pcur)[2][2]) {
    constexpr int q = decltype(qc)::value;  // j mod 4
    BSR_WAIT_VMCNT(kMaxBatchesInFlight * NF);
    __builtin_amdgcn_s_barrier();
    const int32_t nk2 = page_k_fast(j + kKAhead + 1), nv2 = page_v_fast(j + kVAhead + 1);
    dma_kv<NF>(reinterpret_cast<const uint16_t*>(uint64_t(uint32_t(nk)) * page_bytes + k_add),
            lds_k + slot_off((q + kKAhead) & 3),
            reinterpret_cast<const uint16_t*>(uint64_t(uint32_t(nv)) * page_bytes + v_add),
            lds_v + slot_off((q + kVAhead) & 3));
    nk = nk2;
    nv = nv2;
    __builtin_amdgcn_sched_barrier(0);
    const bool any = fused(sl.k0() + slot_off((q + 1) & 3), sl.v0() + slot_off((q + 3) & 3), Snext, Scur, pprev, pcur);
    rescale(any);
  };
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int i = 0; i < 2; ++i) pb[b][i] = u32x4{0u, 0u, 0u, 0u};  // P(-1)
  for (int j = 0;; j += 2) {
    if (j == j_fast) {
      for (int i = 0; i < n_quads; ++i, j += 4) {
        fast_step(Q0{}, j, Sa, Sb, pb, pa);
        fast_step(Q1{}, j + 1, Sb, Sa, pa, pb);
        fast_step(Q2{}, j + 2, Sa, Sb, pb, pa);
        fast_step(Q3{}, j + 3, Sb, Sa, pa, pb);
      }
    }
    step(j, Sa, Sb, pb, pa);
    if (j + 1 > n) break;
    step(j + 1, Sb, Sa, pa, pb);
    if (j + 2 > n) break;
  }

  // ---- epilogue: final output or partial state, per block ----
  acc_settle();
  float inv[2], lse[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float lb = pair_sum(l[b]);  // the two halves of a row held different tokens
    const bool empty = !(lb > 0.f);
    inv[b] = empty ? 0.f : 1.f / lb;
    lse[b] = empty ? kNegInf : (m[b] + log2f(lb)) * kLn2;
  }
  if (item.slot < 0) {
    // The final rows go out through LDS: a lane of the product layout holds 8-byte pieces of 32
    // rows, so stored directly every store instruction would touch 32 partial lines; staged in the
    // (now idle) tile slots, each wave writes its 64 rows back as whole 16-byte row pieces, D / 8
    // lanes per row (for g = 4 one instruction covers the four heads of a query: one contiguous
    // 1 KB run of O).  Rows are padded by 16 bytes against bank conflicts.
    constexpr int RS = 2 * D + 16;  // staging row stride, bytes
    static_assert(128 * RS <= 4 * PF<D>::SLOT, "the staged tile fits in the tile slots");
    lds_u8* st = sl.k0();
    __syncthreads();  // both waves are done with the tile slots
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      lds_u8* rowp = st + (64 * wave + 32 * b + r32) * RS + 8 * h;
#pragma unroll
      for (int cb = 0; cb < KB; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(rowp + 2 * (32 * cb + 8 * q4)) =
              u32x2{cvt_pk_bf16(oacc[b][cb][4 * q4] * inv[b], oacc[b][cb][4 * q4 + 1] * inv[b]),
                    cvt_pk_bf16(oacc[b][cb][4 * q4 + 2] * inv[b], oacc[b][cb][4 * q4 + 3] * inv[b])};
      if (h == 0 && row_ok[b]) a.lse[int64_t(rq.q_start + row_pos[b]) * a.Hq + row_hq[b]] = lse[b];
    }
    __syncthreads();  // (each wave reads back only its own rows; the barrier orders the LDS traffic)
    constexpr int LPR = D / 8, RPI = 64 / LPR;  // lanes per row (16 bytes each), rows per store
    const int sub = lane / LPR, col = 8 * (lane % LPR);
#pragma unroll
    for (int i = 0; i < 64 / RPI; ++i) {
      const int lr = 64 * wave + RPI * i + sub;  // row of the tile
      const int r = item.row_start + lr;
      const u32x4 v = *reinterpret_cast<__attribute__((address_space(3))) const u32x4*>(st + lr * RS + 2 * col);
      if (r < item.row_end) {
        const int64_t orow = int64_t(rq.q_start + r / a.g) * a.Hq + hk * a.g + r % a.g;
        // (streaming: this kernel never reads the rows back)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.o) + orow * D + col));
      }
    }
  } else {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (!row_ok[b]) continue;
      const int r = item.row_start + 64 * wave + 32 * b + r32;
      const int64_t prow = (int64_t(item.slot) * a.Hk + hk) * a.Tq + (r - item.row_start);
      float* pp = a.part_o + prow * D + 4 * h;
#pragma unroll
      for (int cb = 0; cb < KB; ++cb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<f32x4*>(pp + 32 * cb + 8 * q4) =
              f32x4{oacc[b][cb][4 * q4], oacc[b][cb][4 * q4 + 1], oacc[b][cb][4 * q4 + 2], oacc[b][cb][4 * q4 + 3]} *
              inv[b];
      if (h == 0) a.part_lse[prow] = lse[b];
    }
  }
}

}  // namespace

template <int D, int PG, bool VAR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_prefill_bf16_kernel(RunArgs a) {
  constexpr bool POW2 = PG != kPageAny;
  __shared__ __attribute__((aligned(16))) unsigned char lds[Slots<D>::BYTES];
  const Slots<D> sl{(lds_u8*)lds};
  // XCD-aware order: the dispatcher deals consecutive workgroups round-robin to the 8 XCDs,
  // so numbering them KV-head-minor puts every worker of one KV head on the same XCD (for
  // H_kv dividing 8), and the K/V tiles its query tiles share stay in that XCD's L2.
  const int bid = blockIdx.x + gridDim.x * blockIdx.y;
  // (the division runs on the vector ALU; the results are uniform, so read them back as scalars)
  const int hk = __builtin_amdgcn_readfirstlane(bid % a.Hk), w = __builtin_amdgcn_readfirstlane(bid / a.Hk);
  const int it0 = uniform_load(a.qptr + w), it_end = uniform_load(a.qptr + w + 1);
  if (it0 >= it_end) return;
  ItemRec item = uniform_load(a.items + it0);
  for (int it = it0; it < it_end; ++it) {
    RecFetch nf;  // the next item's record, loaded before this item's first tile loads
    nf.load(a.items + it + 1, it + 1 < it_end);
    const ReqRec rq = req_of(a, item);
    const int rows = item.row_end - item.row_start;
    if (rows > 64) prefill_item32<D, true, PG, VAR>(a, item, rq, hk, sl);        // 3-4 blocks of 32 rows, pipelined
    else if (rows > 32) prefill_item32<D, false, PG, VAR>(a, item, rq, hk, sl);  // 2 blocks, tokens split
    else if (rows > 16) prefill_item16<D, 2, POW2, VAR>(a, item, rq, hk, sl);  // 2 blocks of 16 rows
    else prefill_item16<D, 1, POW2, VAR>(a, item, rq, hk, sl);                 // 1 block, tokens split 4 ways
    if (it + 1 < it_end) {
      nf.store(sl.rec());
      __syncthreads();
      item = read_rec(sl.rec());
    }
  }
}

// The 128-row shape: every item of a plan whose query tile is 128 rows.
template <int D, int PG, bool VAR>
__global__ __launch_bounds__(kThreads2) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_prefill128_bf16_kernel(RunArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[Slots<D>::BYTES];
  const Slots<D> sl{(lds_u8*)lds};
  const int bid = blockIdx.x + gridDim.x * blockIdx.y;  // KV-head-minor: see attn_prefill_bf16_kernel
  const int hk = __builtin_amdgcn_readfirstlane(bid % a.Hk), w = __builtin_amdgcn_readfirstlane(bid / a.Hk);
  const int it0 = uniform_load(a.qptr + w), it_end = uniform_load(a.qptr + w + 1);
  if (it0 >= it_end) return;
  ItemRec item = uniform_load(a.items + it0);
  for (int it = it0; it < it_end; ++it) {
    RecFetch nf;
    nf.load(a.items + it + 1, it + 1 < it_end);
    prefill_item128<D, PG, VAR>(a, item, req_of(a, item), hk, sl, nf);
    if (it + 1 < it_end) item = read_rec(sl.rec());
  }
}

bool prefill_bf16_supported(int d, int Tq) { return (d == 64 || d == 128) && Tq % 16 == 0 && Tq <= 128; }

int prefill_bf16_blocks_per_cu(int d) {
  // every page-size variant uses the same resources; ask for one of them
  int nb = 1;
  hipError_t e = hipErrorInvalidValue;
  if (d == 64) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_prefill_bf16_kernel<64, kPageDiv32, false>, kThreads, 0);
  if (d == 128) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_prefill_bf16_kernel<128, kPageDiv32, false>, kThreads, 0);
  return (e == hipSuccess && nb > 0) ? nb : 1;
}

// VAR: the variant instantiations (sliding window, soft cap, custom mask).  Soft-capped plans
// and custom-masked runs use the 4-wave
// shapes for every tile size: their two waves per SIMD overlap the extra exponential and
// reciprocal of each capped score with the other wave's matrix work, where the single wave per
// SIMD of the 128-row shape runs them in series (measured 573 against 542 TFLOP/s on the ragged
// causal prefill with a cap of 50).
template <int D, bool VAR>
static void launch_pg(const RunArgs& a, dim3 grid, hipStream_t s, bool div32, bool pow2) {
  if (a.Tq == 128 && !(VAR && (a.soft_cap > 0.f || a.mask))) {  // 128-row tiles: two waves of two row blocks each
    const dim3 block(kThreads2);
    if (div32) hipLaunchKernelGGL((attn_prefill128_bf16_kernel<D, kPageDiv32, VAR>), grid, block, 0, s, a);
    else if (pow2) hipLaunchKernelGGL((attn_prefill128_bf16_kernel<D, kPagePow2, VAR>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_prefill128_bf16_kernel<D, kPageAny, VAR>), grid, block, 0, s, a);
    return;
  }
  const dim3 block(kThreads);
  if (div32) hipLaunchKernelGGL((attn_prefill_bf16_kernel<D, kPageDiv32, VAR>), grid, block, 0, s, a);
  else if (pow2) hipLaunchKernelGGL((attn_prefill_bf16_kernel<D, kPagePow2, VAR>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((attn_prefill_bf16_kernel<D, kPageAny, VAR>), grid, block, 0, s, a);
}

template <int D>
static void launch_d(const RunArgs& a, dim3 grid, hipStream_t s) {
  const bool div32 = a.p_shift >= 0 && a.P <= 32, pow2 = a.p_shift >= 0;
  if (a.window_left >= 0 || a.soft_cap > 0.f || a.mask) launch_pg<D, true>(a, grid, s, div32, pow2);
  else launch_pg<D, false>(a, grid, s, div32, pow2);
}

hipError_t launch_prefill_bf16(const RunArgs& a, hipStream_t s) {
  dim3 grid(a.C, a.Hk);
  if (a.d == 64) launch_d<64>(a, grid, s);
  else if (a.d == 128) launch_d<128>(a, grid, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bsr
