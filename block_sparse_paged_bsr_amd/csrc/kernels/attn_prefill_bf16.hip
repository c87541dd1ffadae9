// bf16 tiled attention on gfx950 matrix cores: ragged (causal) prefill over a paged
// KV cache, with GQA-packed query tiles.
//
// Data path ("sparse select, dense compute": "FlashInfer: Engineering a
// Customizable, Block-Sparse Attention Engine for LLM Inference Serving" §IV.2 and
// §V.4; "FlashInfer 原理" §⑥): the rows of a 64-token KV tile are looked up through
// the page table (eq. 7 of "FlashInfer: Making Attention Fit the Serving Workload")
// and copied from HBM straight into LDS by 16-byte LDS-DMA loads
// (global_load_lds_dwordx4), in the order the matrix instructions consume them; after
// staging the products are ordinary dense MFMA tiles.  A query tile holds T_q packed
// rows of one KV head (row r -> position floor(r / g), head g * h_kv + r mod g, eq. 3
// of the review), so every staged KV tile serves all g query heads of the group.
//
// LDS layout of one stage (64 tokens): K then V, each as 4 token blocks x D/32 k-blocks
// of 1 KB fragments (64 lanes x 16 bytes, 16 tokens x 32 head-dim values).
//   K fragment: byte 16 L holds K[token L%16][k-block*32 + (L/16)*8 .. +8], exactly the
//               A operand of v_mfma_f32_16x16x32_bf16 for lane L (linear, no conflicts).
//   V fragment: byte 16 L holds V[token (L%32)/2][k-block*32 + (2(L/32) + L%2)*8 .. +8],
//               an order in which every ds_read_b64_tr_b16 of 16 lanes touches each of
//               the 32 LDS banks once.
// Two stages live in two separate LDS arrays: the DMA of tile i+1 into one overlaps the
// products of tile i from the other, and LDS reads never wait for the other stage's DMA.
//
// Per wave, for a 16-row block of packed queries:
//   S^T[token][row] = sum_k K[token][k] Q[row][k]        v_mfma_f32_16x16x32_bf16
//     (A = K fragment, B = Q held in registers for the whole work item;
//      lane n + 16 j receives tokens 4j..4j+3 of row n)
//   online softmax per row in log2 units ("FlashInfer: Engineering ...", §II.2); the
//     reference maximum is raised only when a score exceeds it by more than 8 (so p <= 256),
//     which keeps the result exact (numerator and denominator share the reference) and
//     makes the rescale of the accumulator rare
//   O^T[d][row] += sum_token V^T[d][token] P^T[token][row]  v_mfma_f32_16x16x32_bf16
//     (B = P^T straight from the score accumulators of two 16-token blocks, A = V^T from
//      two transposing reads; both operands use the same token -> k-slot assignment)
//
// Every wave computes all of its row blocks, including an absent second block at the
// end of a request (zero queries, never written), so the products carry no branches.
// Work split inside a workgroup (4 waves): with >= 3 row blocks every wave owns row
// blocks and all 64 tokens of a tile; with 2 (1) row blocks, 2 (4) waves share a
// row block and split the tile's tokens, and their states are combined at the end of
// the item with the merge of eq. 6 (§3.2 of the review).
#include "common.cuh"
#include "launch.h"

namespace bsr {

namespace {

constexpr int kTileKV = 64;  // tokens per staged KV tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleMargin = 8.f;  // log2 units

template <int D>
struct PF {
  static constexpr int KB = D / 32;            // k-blocks per row
  static constexpr int DB = D / 16;            // 16-wide d-blocks of the output
  static constexpr int FRAG = 1024;            // 64 lanes x 16 bytes
  static constexpr int TILE = 4 * KB * FRAG;   // K (or V) of 64 tokens
  static constexpr int STAGE = 2 * TILE;       // K then V
  static constexpr int COMB_WAVE = 16 * (D + 2) * 4;
  static_assert(2 * COMB_WAVE <= STAGE, "combine area must fit in half of the stages");
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

// Issue the LDS-DMA loads of one KV tile (tokens t0 .. t0+63) into `stage`.  Wave w
// loads token block w: D/32 K fragments and D/32 V fragments.  pk / pv are the pages of
// the token this lane carries in a K / V fragment (looked up one tile earlier).
template <int D>
__device__ __forceinline__ void issue_tile(unsigned char* stage, const Paging& pgn, int t0, int32_t pk,
                                           int32_t pv, const uint16_t* K, const uint16_t* V) {
  constexpr int KB = PF<D>::KB;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nk = lane & 15, jk = lane >> 4;
  const int nv = (lane & 31) >> 1, jv = 2 * (lane >> 5) + (lane & 1);
  const uint16_t* kp = K + pgn.row<D>(t0 + w * 16 + nk, pk) + jk * 8;
  const uint16_t* vp = V + pgn.row<D>(t0 + w * 16 + nv, pv) + jv * 8;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    __builtin_amdgcn_global_load_lds(kp + kb * 32, (lds_ptr)(stage + (w * KB + kb) * PF<D>::FRAG), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vp + kb * 32, (lds_ptr)(stage + PF<D>::TILE + (w * KB + kb) * PF<D>::FRAG),
                                     16, 0, 0);
  }
}

template <int D>
__device__ __forceinline__ void tile_pages(const Paging& pgn, int t0, int32_t& pk, int32_t& pv) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  pk = pgn.page_of(t0 + w * 16 + (lane & 15));
  pv = pgn.page_of(t0 + w * 16 + ((lane & 31) >> 1));
}

// One work item.  NRB: row blocks per wave (2 when every wave owns row blocks, else 1);
// NT: 16-token blocks of a tile per wave (4, 2 or 1).
template <int D, int NRB, int NT>
__device__ __forceinline__ void prefill_item(const RunArgs& a, const ItemRec& item, const ReqRec& rq,
                                             int hk, unsigned char* lds0, unsigned char* lds1) {
  constexpr int KB = PF<D>::KB, DB = PF<D>::DB, FRAG = PF<D>::FRAG, TILE = PF<D>::TILE;
  constexpr int N_KS = 4 / NT;  // waves sharing a row block
  constexpr int N_RG = kWaves / N_KS;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, j = lane >> 4;
  const int rg = wave % N_RG, ks = wave / N_RG;
  const int nrows = item.row_end - item.row_start;
  const int RB = (nrows + 15) >> 4;
  const float c = a.sm_scale * kLog2e;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  const int kv_end = item.kv_end;
  const Paging pgn{a.indices, rq.page_start, a.P, a.p_shift, a.Hk, hk, kv_end};

  // row blocks of this wave: rg and rg + N_RG
  bool rb_on[NRB], row_ok[NRB];
  int row_pos[NRB], row_hq[NRB], lim[NRB];
  bf16x8 qb[NRB][KB];
#pragma unroll
  for (int x = 0; x < NRB; ++x) {
    const int rb = rg + x * N_RG;
    rb_on[x] = rb < RB;
    const int r = item.row_start + rb * 16 + n;
    row_ok[x] = rb_on[x] && r < item.row_end;
    row_pos[x] = r / a.g;
    row_hq[x] = hk * a.g + r % a.g;
    lim[x] = kv_end;
    if (a.causal && row_ok[x]) lim[x] = min(kv_end, rq.kv_len - rq.q_len + row_pos[x] + 1);
    const uint16_t* qp = Q + (int64_t(rq.q_start + row_pos[x]) * a.Hq + row_hq[x]) * D + j * 8;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok[x]) v = *reinterpret_cast<const u32x4*>(qp + kb * 32);
      qb[x][kb] = __builtin_bit_cast(bf16x8, v);
    }
  }
  // smallest visible end over the item's rows: tiles ending before it need no mask
  int min_lim = kv_end;
  if (a.causal) min_lim = min(kv_end, rq.kv_len - rq.q_len + item.row_start / a.g + 1);

  float m[NRB], l[NRB];
  f32x4 oacc[NRB][DB];
#pragma unroll
  for (int x = 0; x < NRB; ++x) {
    m[x] = kNegInf;
    l[x] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[x][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // per-lane part of the transposing V read: lane 16G + 4e + q addresses token 4G+e,
  // head-dim values 4q .. 4q+3 of a 16-wide block (see the V fragment order above)
  const int vg = lane >> 4, ve = (lane >> 2) & 3, vq = lane & 3;
  const int vtr_lane = (2 * (4 * vg + ve) + (vq >> 1)) * 16 + 8 * (vq & 1);

  auto compute = [&](const unsigned char* cur, int t0) {
    // ---- scores: each K fragment is read once and used for every row block ----
    f32x4 S[NRB][NT];
#pragma unroll
    for (int x = 0; x < NRB; ++x)
#pragma unroll
      for (int b = 0; b < NT; ++b) S[x][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < NT; ++b) {
      const int tb = ks * NT + b;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(cur + (tb * KB + kb) * FRAG + lane * 16);
#pragma unroll
        for (int x = 0; x < NRB; ++x)
          S[x][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[x][kb], S[x][b], 0, 0, 0);
      }
    }

    // ---- online softmax ----
    const bool need_mask = t0 + kTileKV > min_lim;
    uint32_t pk[NRB][NT][2];
#pragma unroll
    for (int x = 0; x < NRB; ++x) {
      if (need_mask) {
#pragma unroll
        for (int b = 0; b < NT; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = t0 + (ks * NT + b) * 16 + 4 * j + i;
            if (tok >= lim[x]) S[x][b][i] = kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int b = 0; b < NT; ++b) mx = fmaxf(fmaxf(mx, fmaxf(S[x][b][0], S[x][b][1])), fmaxf(S[x][b][2], S[x][b][3]));
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mxs = mx * c;
      const bool raise = mxs > m[x] + kRescaleMargin;
      if (__ballot(raise)) {  // wave-uniform: rare once the row maxima have settled
        const float mnew = raise ? mxs : m[x];
        const float corr = fast_exp2(m[x] - (mnew == kNegInf ? 0.f : mnew));
        l[x] *= corr;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[x][db] *= corr;
        m[x] = mnew;
      }
      const float muse = m[x] == kNegInf ? 0.f : m[x];
      float lsum = 0.f;
#pragma unroll
      for (int b = 0; b < NT; ++b) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = fast_exp2(__builtin_fmaf(S[x][b][i], c, -muse));
          lsum += p[i];
        }
        pk[x][b][0] = cvt_pk_bf16(p[0], p[1]);
        pk[x][b][1] = cvt_pk_bf16(p[2], p[3]);
      }
      l[x] += lsum;
    }

    // ---- O^T += V^T P^T: each V fragment is read once and used for every row block ----
    const unsigned char* vt = cur + TILE + vtr_lane;
    if constexpr (NT >= 2) {
#pragma unroll
      for (int b = 0; b < NT; b += 2) {
        const int tba = ks * NT + b, tbb = tba + 1;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int off = (db >> 1) * FRAG + (db & 1) * 512;
          const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vt + tba * KB * FRAG + off));
          const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vt + tbb * KB * FRAG + off));
          const bf16x8 vab = __builtin_bit_cast(
              bf16x8, u32x4{__builtin_bit_cast(u32x2, va)[0], __builtin_bit_cast(u32x2, va)[1],
                            __builtin_bit_cast(u32x2, vb)[0], __builtin_bit_cast(u32x2, vb)[1]});
#pragma unroll
          for (int x = 0; x < NRB; ++x) {
            const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[x][b][0], pk[x][b][1], pk[x][b + 1][0], pk[x][b + 1][1]});
            oacc[x][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vab, pb, oacc[x][db], 0, 0, 0);
          }
        }
      }
    } else {
      const int tb = ks;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int off = (db >> 1) * FRAG + (db & 1) * 512;
        const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(vt + tb * KB * FRAG + off));
#pragma unroll
        for (int x = 0; x < NRB; ++x) {
          const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{pk[x][0][0], pk[x][0][1]});
          oacc[x][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[x][db], 0, 0, 0);
        }
      }
    }
  };

  // ---- tile loop: DMA of tile i+1 overlaps the products of tile i ----
  const int ntiles = (kv_end - item.kv_start + kTileKV - 1) / kTileKV;
  int32_t pk_next, pv_next;
  __syncthreads();  // LDS free (previous item finished, including its combine)
  tile_pages<D>(pgn, item.kv_start, pk_next, pv_next);
  issue_tile<D>(lds0, pgn, item.kv_start, pk_next, pv_next, K, V);
  tile_pages<D>(pgn, item.kv_start + kTileKV, pk_next, pv_next);
  __syncthreads();  // waits for this wave's DMA, then for every wave's
  for (int ti = 0; ti < ntiles; ti += 2) {
    const int t0 = item.kv_start + ti * kTileKV;
    if (ti + 1 < ntiles) {
      issue_tile<D>(lds1, pgn, t0 + kTileKV, pk_next, pv_next, K, V);
      tile_pages<D>(pgn, t0 + 2 * kTileKV, pk_next, pv_next);
    }
    compute(lds0, t0);
    __syncthreads();
    if (ti + 1 < ntiles) {
      if (ti + 2 < ntiles) {
        issue_tile<D>(lds0, pgn, t0 + 2 * kTileKV, pk_next, pv_next, K, V);
        tile_pages<D>(pgn, t0 + 3 * kTileKV, pk_next, pv_next);
      }
      compute(lds1, t0 + kTileKV);
      __syncthreads();
    }
  }

  // row sums: each lane held the sum over its own tokens
#pragma unroll
  for (int x = 0; x < NRB; ++x) {
    l[x] += shfl_xor(l[x], 16);
    l[x] += shfl_xor(l[x], 32);
  }

  if constexpr (N_KS > 1) {
    // combine the waves that split this row block's tokens (one row block each);
    // waves 0-1 use the first stage's array, waves 2-3 the second one's
    auto comb_of = [&](int wv) -> float* {
      return reinterpret_cast<float*>((wv < 2 ? lds0 : lds1) + (wv & 1) * PF<D>::COMB_WAVE);
    };
    float* mine = comb_of(wave);
    if (rb_on[0]) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[n * (D + 2) + db * 16 + 4 * j + i] = oacc[0][db][i];
      if (j == 0) {
        mine[n * (D + 2) + D] = m[0];
        mine[n * (D + 2) + D + 1] = l[0];
      }
    }
    __syncthreads();
    if (ks == 0 && rb_on[0]) {
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
          oacc[0][db][i] = sum;
        }
      m[0] = mm;
      l[0] = lt;
    }
  }

  // ---- epilogue: final output or partial state ----
  if (ks == 0) {
    uint16_t* __restrict__ O = static_cast<uint16_t*>(a.o);
#pragma unroll
    for (int x = 0; x < NRB; ++x) {
      if (!row_ok[x]) continue;
      const int r = item.row_start + (rg + x * N_RG) * 16 + n;
      const bool empty = !(l[x] > 0.f);
      const float inv = empty ? 0.f : 1.f / l[x];
      const float lse = empty ? kNegInf : (m[x] + log2f(l[x])) * kLn2;
      if (item.slot < 0) {
        const int64_t orow = int64_t(rq.q_start + row_pos[x]) * a.Hq + row_hq[x];
        uint16_t* op = O + orow * D + 4 * j;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const f32x4 v = oacc[x][db] * inv;
          *reinterpret_cast<u32x2*>(op + db * 16) = u32x2{cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3])};
        }
        if (j == 0) a.lse[orow] = lse;
      } else {
        const int64_t prow = (int64_t(item.slot) * a.Hk + hk) * a.Tq + (r - item.row_start);
        float* pp = a.part_o + prow * D + 4 * j;
#pragma unroll
        for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(pp + db * 16) = oacc[x][db] * inv;
        if (j == 0) a.part_lse[prow] = lse;
      }
    }
  }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_prefill_bf16_kernel(RunArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds0[PF<D>::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[PF<D>::STAGE];
  const int w = blockIdx.x, hk = blockIdx.y;
  for (int it = a.qptr[w]; it < a.qptr[w + 1]; ++it) {
    const ItemRec item = a.items[it];
    const ReqRec rq = a.req[item.req];
    const int RB = (item.row_end - item.row_start + 15) >> 4;
    if (RB >= 3) prefill_item<D, 2, 4>(a, item, rq, hk, lds0, lds1);
    else if (RB == 2) prefill_item<D, 1, 2>(a, item, rq, hk, lds0, lds1);
    else prefill_item<D, 1, 1>(a, item, rq, hk, lds0, lds1);
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
