// bf16 tiled attention on gfx950 matrix cores: ragged (causal) prefill over a paged
// KV cache, with GQA-packed query tiles.
//
// Data path ("sparse select, dense compute": "FlashInfer: Engineering a
// Customizable, Block-Sparse Attention Engine for LLM Inference Serving" §IV.2 and
// §V.4; "FlashInfer 原理" §⑥): the rows of a 64-token KV tile are looked up through
// the page table (eq. 7 of "FlashInfer: Making Attention Fit the Serving Workload")
// and staged into LDS with 16-byte loads, K and V both as [token][d]; after staging
// the products are ordinary dense MFMA tiles.  A query tile holds T_q packed rows of
// one KV head (row r -> position floor(r / g), head g * h_kv + r mod g, eq. 3 of the
// review), so every staged KV tile serves all g query heads of the group.
//
// Per wave, for a 16-row block of packed queries:
//   S^T[token][row] = sum_k K[token][k] Q[row][k]        v_mfma_f32_16x16x32_bf16
//     (A = K rows read from LDS, B = Q held in registers for the whole work item;
//      lane n + 16 j receives tokens 4j..4j+3 of row n)
//   online softmax per row in log2 units ("FlashInfer: Engineering ...", §II.2)
//   O^T[d][row] += sum_token V^T[d][token] P^T[token][row]  v_mfma_f32_16x16x32_bf16
//     (B = P^T straight from the score accumulators of two 16-token blocks, A = V^T
//      from ds_read_b64_tr_b16 transposing reads of the same two blocks; both operands
//      use the same token -> k-slot assignment, so the product sums over the tokens)
// The next KV tile is fetched from HBM into registers while the current one is
// computed, and written to the second LDS buffer afterwards (one barrier per tile).
//
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

template <int D>
struct PrefillSmem {
  static constexpr int RS = D + 8;  // row stride (elements): 16-byte aligned, rows offset by 4 banks
  static constexpr int TILE_BYTES = kTileKV * RS * 2;  // one K or V tile
  static constexpr int BUF_BYTES = 2 * TILE_BYTES;     // K + V
  static constexpr int COMB_BYTES = kWaves * 16 * (D + 2) * 4;
  static constexpr int BYTES = (2 * BUF_BYTES) > COMB_BYTES ? (2 * BUF_BYTES) : COMB_BYTES;
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  bf16x2 r;
  r[0] = static_cast<__bf16>(a);
  r[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct Stage {
  static constexpr int CH = D / 8;                      // 16-byte chunks per row
  static constexpr int PER_THREAD = kTileKV * CH / kThreads;
  u32x4 k[PER_THREAD], v[PER_THREAD];
};

// Fetch one KV tile (tokens t0 .. t0+63 of the request, clamped to the chunk end) into
// registers: thread tid handles chunk tid % CH of tokens tid / CH + (kThreads / CH) u.
template <int D>
__device__ __forceinline__ void fetch_tile(Stage<D>& st, const RunArgs& a, const ReqRec& rq, int hk,
                                           int t0, int kv_end, int tid, const uint16_t* __restrict__ K,
                                           const uint16_t* __restrict__ V) {
  constexpr int CH = Stage<D>::CH;
#pragma unroll
  for (int u = 0; u < Stage<D>::PER_THREAD; ++u) {
    const int idx = tid + u * kThreads;
    const int tt = idx / CH, ch = idx % CH;
    const int tok = min(t0 + tt, kv_end - 1);  // clamped rows are masked, never read out of range
    const int64_t base = (page_row(a.indices, rq.page_start, tok, a.P, a.p_shift) * a.Hk + hk) * D + ch * 8;
    st.k[u] = *reinterpret_cast<const u32x4*>(K + base);
    st.v[u] = *reinterpret_cast<const u32x4*>(V + base);
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const Stage<D>& st, uint16_t* Ks, uint16_t* Vs, int tid) {
  constexpr int CH = Stage<D>::CH;
  constexpr int RS = PrefillSmem<D>::RS;
#pragma unroll
  for (int u = 0; u < Stage<D>::PER_THREAD; ++u) {
    const int idx = tid + u * kThreads;
    const int tt = idx / CH, ch = idx % CH;
    *reinterpret_cast<u32x4*>(Ks + tt * RS + ch * 8) = st.k[u];
    *reinterpret_cast<u32x4*>(Vs + tt * RS + ch * 8) = st.v[u];
  }
}

// One work item.  NRB: row blocks per wave (2 when every wave owns row blocks, else 1);
// NT: 16-token blocks of a tile per wave (4, 2 or 1).
template <int D, int NRB, int NT>
__device__ __forceinline__ void prefill_item(const RunArgs& a, const ItemRec& item, const ReqRec& rq,
                                             int hk, unsigned char* smem) {
  using SM = PrefillSmem<D>;
  constexpr int KB = D / 32, DB = D / 16, RS = SM::RS;
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

  // row blocks of this wave: rg and rg + N_RG
  bool rb_on[NRB], row_ok[NRB];
  int row_pos[NRB], row_hq[NRB], lim[NRB];
  bf16x8 qb[NRB][KB];
  int min_lim = kv_end;
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
  if (a.causal) {
    const int first_pos = item.row_start / a.g;
    min_lim = min(kv_end, rq.kv_len - rq.q_len + first_pos + 1);
  }

  float m[NRB], l[NRB];
  f32x4 oacc[NRB][DB];
#pragma unroll
  for (int x = 0; x < NRB; ++x) {
    m[x] = kNegInf;
    l[x] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[x][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int ntiles = (kv_end - item.kv_start + kTileKV - 1) / kTileKV;
  Stage<D> st;
  __syncthreads();  // LDS free (previous item finished, including its combine)
  fetch_tile<D>(st, a, rq, hk, item.kv_start, kv_end, tid, K, V);
  store_tile<D>(st, reinterpret_cast<uint16_t*>(smem), reinterpret_cast<uint16_t*>(smem + SM::TILE_BYTES), tid);
  __syncthreads();

  for (int ti = 0; ti < ntiles; ++ti) {
    const int t0 = item.kv_start + ti * kTileKV;
    unsigned char* buf = smem + (ti & 1) * SM::BUF_BYTES;
    const uint16_t* Ks = reinterpret_cast<const uint16_t*>(buf);
    const uint16_t* Vs = reinterpret_cast<const uint16_t*>(buf + SM::TILE_BYTES);
    const bool has_next = ti + 1 < ntiles;
    if (has_next) fetch_tile<D>(st, a, rq, hk, t0 + kTileKV, kv_end, tid, K, V);

    // ---- scores: K fragments read once, used for every row block ----
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
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (tb * 16 + n) * RS + kb * 32 + j * 8);
#pragma unroll
        for (int x = 0; x < NRB; ++x)
          if (rb_on[x]) S[x][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[x][kb], S[x][b], 0, 0, 0);
      }
    }

    // ---- online softmax ----
    const bool need_mask = t0 + kTileKV > min_lim;
    uint32_t pk[NRB][NT][2];
#pragma unroll
    for (int x = 0; x < NRB; ++x) {
      if (!rb_on[x]) continue;
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
      const float mnew = fmaxf(m[x], mx * c);
      const float muse = mnew == kNegInf ? 0.f : mnew;
      const float corr = fast_exp2(m[x] - muse);
      m[x] = mnew;
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
      l[x] = l[x] * corr + lsum;
      if (corr != 1.f) {
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[x][db] *= corr;
      }
    }

    // ---- O^T += V^T P^T: V fragments read once, used for every row block ----
    // ds_read_b64_tr_b16: lane 16G+i receives V[token 4G+e][d0+i], e = 0..3, when lane
    // 16G+4e+q addresses V[token 4G+e][d0 + 4q .. +4].
    const uint16_t* vtr = Vs + (4 * j + ((lane >> 2) & 3)) * RS + 4 * (lane & 3);
    if constexpr (NT >= 2) {
#pragma unroll
      for (int b = 0; b < NT; b += 2) {
        const int tba = ks * NT + b, tbb = tba + 1;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(vtr + tba * 16 * RS + db * 16));
          const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(vtr + tbb * 16 * RS + db * 16));
          const bf16x8 vab = __builtin_bit_cast(
              bf16x8, u32x4{__builtin_bit_cast(u32x2, va)[0], __builtin_bit_cast(u32x2, va)[1],
                            __builtin_bit_cast(u32x2, vb)[0], __builtin_bit_cast(u32x2, vb)[1]});
#pragma unroll
          for (int x = 0; x < NRB; ++x) {
            if (!rb_on[x]) continue;
            const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[x][b][0], pk[x][b][1], pk[x][b + 1][0], pk[x][b + 1][1]});
            oacc[x][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vab, pb, oacc[x][db], 0, 0, 0);
          }
        }
      }
    } else {
      const int tb = ks;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vtr + tb * 16 * RS + db * 16));
#pragma unroll
        for (int x = 0; x < NRB; ++x) {
          if (!rb_on[x]) continue;
          const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{pk[x][0][0], pk[x][0][1]});
          oacc[x][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[x][db], 0, 0, 0);
        }
      }
    }

    if (has_next) {
      unsigned char* nbuf = smem + ((ti + 1) & 1) * SM::BUF_BYTES;
      store_tile<D>(st, reinterpret_cast<uint16_t*>(nbuf), reinterpret_cast<uint16_t*>(nbuf + SM::TILE_BYTES), tid);
    }
    __syncthreads();
  }

  // row sums: each lane held the sum over its own tokens
#pragma unroll
  for (int x = 0; x < NRB; ++x) {
    l[x] += shfl_xor(l[x], 16);
    l[x] += shfl_xor(l[x], 32);
  }

  if constexpr (N_KS > 1) {
    // combine the waves that split this row block's tokens (one row block each)
    float* comb = reinterpret_cast<float*>(smem);
    float* mine = comb + wave * 16 * (D + 2);
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
      for (int o = 0; o < N_KS; ++o) mm = fmaxf(mm, comb[(rg + o * N_RG) * 16 * (D + 2) + n * (D + 2) + D]);
      const float muse = mm == kNegInf ? 0.f : mm;
      float lt = 0.f, wgt[N_KS];
#pragma unroll
      for (int o = 0; o < N_KS; ++o) {
        const float* src = comb + (rg + o * N_RG) * 16 * (D + 2) + n * (D + 2);
        wgt[o] = fast_exp2(src[D] - muse);
        lt += wgt[o] * src[D + 1];
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sum = 0.f;
#pragma unroll
          for (int o = 0; o < N_KS; ++o)
            sum += wgt[o] * comb[(rg + o * N_RG) * 16 * (D + 2) + n * (D + 2) + db * 16 + 4 * j + i];
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
  using SM = PrefillSmem<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::BYTES];
  const int w = blockIdx.x, hk = blockIdx.y;
  for (int it = a.qptr[w]; it < a.qptr[w + 1]; ++it) {
    const ItemRec item = a.items[it];
    const ReqRec rq = a.req[item.req];
    const int RB = (item.row_end - item.row_start + 15) >> 4;
    if (RB >= 3) prefill_item<D, 2, 4>(a, item, rq, hk, smem);
    else if (RB == 2) prefill_item<D, 1, 2>(a, item, rq, hk, smem);
    else prefill_item<D, 1, 1>(a, item, rq, hk, smem);
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
