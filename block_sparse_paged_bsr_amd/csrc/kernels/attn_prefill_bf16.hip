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
// LDS layout of one stage (64 tokens): K then V, each as 4 token groups (16 tokens) x
// D/32 column groups (32 head-dim values) of 1 KB fragments, 64 lanes x 16 bytes:
//   K fragment (a, b): byte 16 L holds K[16a + L%16][32b + 8(L/16) .. +8]
//   V fragment (a, b): byte 16 L holds V[16a + t][32b + 8c .. +8], c = L/16,
//                      t = (L%16) xor 4(c%2)
// Every DMA instruction reads 64 contiguous bytes of 16 token rows.  The swizzle of the
// V fragments makes each ds_read_b64_tr_b16 (16 lanes x 8 bytes) hit the 32 LDS banks
// once, for both matrix shapes below; K reads are linear or one 256-byte row apart.
// Two stages live in two separate LDS arrays: the DMA of tile i+1 into one overlaps the
// products of tile i from the other, and LDS reads never wait for the other stage's DMA.
//
// Large query tiles (more than 32 packed rows) use v_mfma_f32_32x32x16_bf16 (on gfx950
// it sustains about twice the rate of the 16x16x32 shape).  Per wave, a 32-row block:
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
// Small query tiles (at most 32 rows: decode-like and short requests, the composable
// prefix level) use the 16x16x32 shape with 16-row blocks.
//
// Every wave computes all of its row blocks, including absent ones at the end of a
// request (zero queries, never written), so the products carry no branches.  When a
// tile has fewer row blocks than waves, waves also split the tile's tokens and their
// states are combined at the end of the item with the merge of eq. 6 (§3.2 of the
// review).
#include "common.cuh"
#include "launch.h"

namespace bsr {

namespace {

constexpr int kTileKV = 64;  // tokens per staged KV tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleMargin = 8.f;  // log2 units

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int D>
struct PF {
  static constexpr int KB = D / 32;           // 32-wide column groups per row
  static constexpr int FRAG = 1024;           // 64 lanes x 16 bytes
  static constexpr int TILE = 4 * KB * FRAG;  // K (or V) of 64 tokens
  static constexpr int STAGE = 2 * TILE;      // K then V
  static constexpr int COMB16 = 16 * (D + 2) * 4;  // combine area of one 16-row wave
  static constexpr int COMB32 = 32 * (D + 2) * 4;  // combine area of one 32-row wave
  static_assert(2 * COMB16 <= STAGE && COMB32 <= STAGE, "combine areas must fit in the stages");
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  bf16x2 r;
  r[0] = static_cast<__bf16>(a);
  r[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

__device__ __forceinline__ s16x4 tr_read(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(p));
}

__device__ __forceinline__ bf16x8 cat(s16x4 lo, s16x4 hi) {
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// byte offset, inside a V fragment, of the 8-byte chunk c (head-dim 4c .. 4c+3 of the
// fragment's 32 columns) of token t (0..15)
__device__ __forceinline__ int v_chunk(int t, int c) {
  const int c16 = c >> 1;
  return 16 * (16 * c16 + (t ^ (4 * (c16 & 1)))) + 8 * (c & 1);
}

struct Paging {
  const int32_t* indices;
  int32_t page_start, P, p_shift, Hk, hk, kv_end;
  __device__ __forceinline__ int32_t page_of(int t) const {
    const int tc = min(t, kv_end - 1);
    return indices[page_start + (p_shift >= 0 ? (tc >> p_shift) : tc / P)];
  }
  // first element of token t's row for this KV head, t clamped to the chunk
  template <int D>
  __device__ __forceinline__ int64_t row(int t, int32_t page) const {
    const int tc = min(t, kv_end - 1);
    const int off = p_shift >= 0 ? (tc & ((1 << p_shift) - 1)) : tc - (tc / P) * P;
    return ((int64_t(page) * P + off) * Hk + hk) * D;
  }
};

// tokens (within the wave's 16-token group) carried by this lane in K / V fragments
__device__ __forceinline__ int k_dma_token(int lane) { return lane & 15; }
__device__ __forceinline__ int v_dma_token(int lane) { return (lane & 15) ^ ((lane >> 2) & 4); }

// Issue the LDS-DMA loads of one KV tile (tokens t0 .. t0+63) into `stage`.  Wave w
// loads token group w: D/32 K fragments and D/32 V fragments.  pk / pv are the pages of
// the tokens this lane carries (looked up one tile earlier).
template <int D>
__device__ __forceinline__ void issue_tile(unsigned char* stage, const Paging& pgn, int t0, int32_t pk,
                                           int32_t pv, const uint16_t* K, const uint16_t* V) {
  constexpr int KB = PF<D>::KB;
  // the wave index is read as a scalar so the LDS destinations (M0) are formed on the SALU
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint16_t* kp = K + pgn.row<D>(t0 + w * 16 + k_dma_token(lane), pk) + 8 * (lane >> 4);
  const uint16_t* vp = V + pgn.row<D>(t0 + w * 16 + v_dma_token(lane), pv) + 8 * (lane >> 4);
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    __builtin_amdgcn_global_load_lds(kp + b * 32, (lds_ptr)(stage + (w * KB + b) * PF<D>::FRAG), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vp + b * 32, (lds_ptr)(stage + PF<D>::TILE + (w * KB + b) * PF<D>::FRAG),
                                     16, 0, 0);
  }
}

__device__ __forceinline__ void tile_pages(const Paging& pgn, int t0, int32_t& pk, int32_t& pv) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  pk = pgn.page_of(t0 + w * 16 + k_dma_token(lane));
  pv = pgn.page_of(t0 + w * 16 + v_dma_token(lane));
}

// The double-buffered tile loop shared by both paths: compute(stage, t0) is called once
// per 64-token tile while the next tile's DMA is in flight.
template <int D, typename F>
__device__ __forceinline__ void tile_loop(const Paging& pgn, int kv_start, int kv_end, unsigned char* lds0,
                                          unsigned char* lds1, const uint16_t* K, const uint16_t* V, F&& compute) {
  const int ntiles = (kv_end - kv_start + kTileKV - 1) / kTileKV;
  int32_t pk, pv;
  __syncthreads();  // LDS free (previous item finished, including its combine)
  tile_pages(pgn, kv_start, pk, pv);
  issue_tile<D>(lds0, pgn, kv_start, pk, pv, K, V);
  tile_pages(pgn, kv_start + kTileKV, pk, pv);
  __syncthreads();  // waits for this wave's DMA, then for every wave's
  for (int ti = 0; ti < ntiles; ti += 2) {
    const int t0 = kv_start + ti * kTileKV;
    if (ti + 1 < ntiles) {
      issue_tile<D>(lds1, pgn, t0 + kTileKV, pk, pv, K, V);
      tile_pages(pgn, t0 + 2 * kTileKV, pk, pv);
    }
    compute(static_cast<const unsigned char*>(lds0), t0);
    __syncthreads();
    if (ti + 1 < ntiles) {
      if (ti + 2 < ntiles) {
        issue_tile<D>(lds0, pgn, t0 + 2 * kTileKV, pk, pv, K, V);
        tile_pages(pgn, t0 + 3 * kTileKV, pk, pv);
      }
      compute(static_cast<const unsigned char*>(lds1), t0 + kTileKV);
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
// Large query tiles: 32-row blocks on v_mfma_f32_32x32x16_bf16.
// NT32: 32-token blocks of a tile per wave (2: the whole tile, 1: half, the other half
// goes to a second wave sharing the row block).
// ---------------------------------------------------------------------------------
template <int D, int NT32>
__device__ __forceinline__ void prefill_item32(const RunArgs& a, const ItemRec& item, const ReqRec& rq, int hk,
                                               unsigned char* lds0, unsigned char* lds1) {
  constexpr int KB = PF<D>::KB, FRAG = PF<D>::FRAG, TILE = PF<D>::TILE;
  constexpr int KS16 = D / 16;  // 16-deep k-steps of the score product
  constexpr int N_KS = 2 / NT32;
  constexpr int N_RG = kWaves / N_KS;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r32 = lane & 31, h = lane >> 5;
  const int rg = wave % N_RG, ks = wave / N_RG;
  const int nrows = item.row_end - item.row_start;
  const float c = a.sm_scale * kLog2e;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  const int kv_end = item.kv_end;
  const Paging pgn{a.indices, rq.page_start, a.P, a.p_shift, a.Hk, hk, kv_end};

  // this lane's query row: block rg, row r32
  const int r = item.row_start + rg * 32 + r32;
  const bool rb_on = rg * 32 < nrows;
  const bool row_ok = r < item.row_end;
  const int row_pos = r / a.g, row_hq = hk * a.g + r % a.g;
  const int lim = (a.causal && row_ok) ? min(kv_end, rq.kv_len - rq.q_len + row_pos + 1) : kv_end;
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

  float m = kNegInf, l = 0.f;
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

  auto compute = [&](const unsigned char* cur, int t0) {
    f32x16 S[NT32];
#pragma unroll
    for (int b = 0; b < NT32; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) S[b][i] = 0.f;
#pragma unroll
    for (int k = 0; k < KS16; ++k) {
#pragma unroll
      for (int b = 0; b < NT32; ++b) {
        const int tb = ks * NT32 + b;  // 32-token block of the tile
        const int grp = 2 * tb + (r32 >> 4);
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(cur + (grp * KB + (k >> 1)) * FRAG + k_pos + 512 * (k & 1));
        S[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[k], S[b], 0, 0, 0);
      }
    }
    if (t0 + kTileKV > min_lim) {
#pragma unroll
      for (int b = 0; b < NT32; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = t0 + 32 * (ks * NT32 + b) + 8 * (i >> 2) + 4 * h + (i & 3);
          if (tok >= lim) S[b][i] = kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int b = 0; b < NT32; ++b)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(S[b][i], S[b][i + 1]));
    mx = pair_max(mx);
    bool any;
    const float corr = raise_reference(m, mx * c, any);
    if (any) {
      l *= corr;
#pragma unroll
      for (int b = 0; b < KB; ++b) oacc[b] *= corr;
    }
    const float muse = m == kNegInf ? 0.f : m;
    uint32_t pk[NT32][8];
    float lsum = 0.f;
#pragma unroll
    for (int b = 0; b < NT32; ++b)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(S[b][i], c, -muse));
        const float p1 = fast_exp2(__builtin_fmaf(S[b][i + 1], c, -muse));
        lsum += p0 + p1;
        pk[b][i >> 1] = cvt_pk_bf16(p0, p1);
      }
    l += lsum;
    // O^T += V^T P^T, one 16-token k-block kb at a time
#pragma unroll
    for (int b = 0; b < NT32; ++b)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int grp = 2 * (ks * NT32 + b) + half;  // 16-token group of the tile
        const bf16x8 pb = __builtin_bit_cast(
            bf16x8, u32x4{pk[b][4 * half], pk[b][4 * half + 1], pk[b][4 * half + 2], pk[b][4 * half + 3]});
        const unsigned char* vf = cur + TILE + grp * KB * FRAG;
#pragma unroll
        for (int cb = 0; cb < KB; ++cb) {
          const bf16x8 va = cat(tr_read(vf + cb * FRAG + v_lo), tr_read(vf + cb * FRAG + v_hi));
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[cb], 0, 0, 0);
        }
      }
  };
  tile_loop<D>(pgn, item.kv_start, kv_end, lds0, lds1, K, V, compute);

  l = pair_sum(l);  // the two halves of a row held different tokens

  if constexpr (N_KS > 1) {
    // combine the two waves that split each row block's tokens: the second one publishes
    // its state, the first one folds it in
    float* comb = reinterpret_cast<float*>(rg == 0 ? lds0 : lds1);
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
template <int D, int NT>
__device__ __forceinline__ void prefill_item16(const RunArgs& a, const ItemRec& item, const ReqRec& rq, int hk,
                                               unsigned char* lds0, unsigned char* lds1) {
  constexpr int KB = PF<D>::KB, DB = D / 16, FRAG = PF<D>::FRAG, TILE = PF<D>::TILE;
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
  const Paging pgn{a.indices, rq.page_start, a.P, a.p_shift, a.Hk, hk, kv_end};

  const int r = item.row_start + rg * 16 + n;
  const bool rb_on = rg * 16 < nrows;
  const bool row_ok = r < item.row_end;
  const int row_pos = r / a.g, row_hq = hk * a.g + r % a.g;
  const int lim = (a.causal && row_ok) ? min(kv_end, rq.kv_len - rq.q_len + row_pos + 1) : kv_end;
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

  auto compute = [&](const unsigned char* cur, int t0) {
    f32x4 S[NT];
#pragma unroll
    for (int b = 0; b < NT; ++b) S[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const int tb = ks * NT + b;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(cur + (tb * KB + kb) * FRAG + lane * 16);
        S[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[kb], S[b], 0, 0, 0);
      }
    }
    if (t0 + kTileKV > min_lim) {
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
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(__builtin_fmaf(S[b][i], c, -muse));
        lsum += p[i];
      }
      pk[b][0] = cvt_pk_bf16(p[0], p[1]);
      pk[b][1] = cvt_pk_bf16(p[2], p[3]);
    }
    l += lsum;
    if constexpr (NT >= 2) {
#pragma unroll
      for (int b = 0; b < NT; b += 2) {
        const int tba = ks * NT + b, tbb = tba + 1;
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[b][0], pk[b][1], pk[b + 1][0], pk[b + 1][1]});
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int off = TILE + (db >> 1) * FRAG + ((db & 1) ? v_odd : v_even);
          const bf16x8 vab = cat(tr_read(cur + tba * KB * FRAG + off), tr_read(cur + tbb * KB * FRAG + off));
          oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vab, pb, oacc[db], 0, 0, 0);
        }
      }
    } else {
      const int tb = ks;
      const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{pk[0][0], pk[0][1]});
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int off = TILE + (db >> 1) * FRAG + ((db & 1) ? v_odd : v_even);
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(tr_read(cur + tb * KB * FRAG + off), pb, oacc[db], 0, 0, 0);
      }
    }
  };
  tile_loop<D>(pgn, item.kv_start, kv_end, lds0, lds1, K, V, compute);

  l = pair16_sum(l);
  l = pair_sum(l);

  {
    // combine the waves that split this row block's tokens; waves 0-1 use the first
    // stage's array, waves 2-3 the second one's
    auto comb_of = [&](int wv) -> float* {
      return reinterpret_cast<float*>((wv < 2 ? lds0 : lds1) + (wv & 1) * PF<D>::COMB16);
    };
    float* mine = comb_of(wave);
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
        const float* src = comb_of(rg + o * N_RG) + n * (D + 2);
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

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_prefill_bf16_kernel(RunArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds0[PF<D>::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[PF<D>::STAGE];
  // XCD-aware order: the dispatcher deals consecutive workgroups round-robin to the 8 XCDs,
  // so numbering them KV-head-minor puts every worker of one KV head on the same XCD (for
  // H_kv dividing 8), and the K/V tiles its query tiles share stay in that XCD's L2.
  const int bid = blockIdx.x + gridDim.x * blockIdx.y;
  const int hk = bid % a.Hk, w = bid / a.Hk;
  for (int it = a.qptr[w]; it < a.qptr[w + 1]; ++it) {
    const ItemRec item = a.items[it];
    const ReqRec rq = a.req[item.req];
    const int rows = item.row_end - item.row_start;
    if (rows > 64) prefill_item32<D, 2>(a, item, rq, hk, lds0, lds1);       // 3-4 blocks of 32 rows
    else if (rows > 32) prefill_item32<D, 1>(a, item, rq, hk, lds0, lds1);  // 2 blocks, tokens split
    else if (rows > 16) prefill_item16<D, 2>(a, item, rq, hk, lds0, lds1);  // 2 blocks of 16 rows
    else prefill_item16<D, 1>(a, item, rq, hk, lds0, lds1);                 // 1 block, tokens split 4 ways
  }
}

bool prefill_bf16_supported(int d, int Tq) { return (d == 64 || d == 128) && Tq % 16 == 0 && Tq <= 128; }

int prefill_bf16_blocks_per_cu(int d) {
  int nb = 1;
  hipError_t e = hipErrorInvalidValue;
  if (d == 64) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_prefill_bf16_kernel<64>, kThreads, 0);
  if (d == 128) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_prefill_bf16_kernel<128>, kThreads, 0);
  return (e == hipSuccess && nb > 0) ? nb : 1;
}

hipError_t launch_prefill_bf16(const RunArgs& a, hipStream_t s) {
  dim3 grid(a.C, a.Hk), block(kThreads);
  if (a.d == 64) hipLaunchKernelGGL(attn_prefill_bf16_kernel<64>, grid, block, 0, s, a);
  else if (a.d == 128) hipLaunchKernelGGL(attn_prefill_bf16_kernel<128>, grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bsr
