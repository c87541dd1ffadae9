// bf16 tiled attention on gfx950 matrix cores: ragged (causal) prefill over a paged
// KV cache, with GQA-packed query tiles.
//
// Data path ("sparse select, dense compute": "FlashInfer: Engineering a
// Customizable, Block-Sparse Attention Engine for LLM Inference Serving" §IV.2 and
// §V.4; "FlashInfer 原理" §⑥): the rows of a 64-token KV tile are looked up through
// the page table (eq. 7 of "FlashInfer: Making Attention Fit the Serving Workload")
// and staged into LDS with 16-byte loads -- K as [token][d], V transposed as
// [d][token] -- after which the score and output products are ordinary dense MFMA
// tiles.  A query tile holds T_q packed rows of one KV head (row r -> position
// floor(r / g), head g * h_kv + r mod g, eq. 3), so every staged KV tile serves all g
// query heads of the group.
//
// Per wave, for a 16-row block of packed queries and a 16-token block of keys:
//   S^T[token][row] = sum_k K[token][k] Q[row][k]       v_mfma_f32_16x16x32_bf16
//   online softmax over tokens, per row, in log2 units ("FlashInfer: Engineering ...",
//   §II.2; the exponent base change is exact up to rounding)
//   O^T[d][row] += sum_token V^T[d][token] P^T[token][row]  v_mfma_f32_16x16x16_bf16
// Computing the transposed products lets the fp32 score accumulator (lane holds
// tokens 4*(lane/16)+i of row lane%16) feed the next product's B operand directly.
//
// Work split inside a workgroup (4 waves): with >= 4 row blocks every wave owns
// row blocks; with fewer, waves also split the 64-token KV tile and their states are
// combined at the end of the item with the merge of eq. 6 (§3.2 of the review).
#include "common.cuh"
#include "launch.h"

namespace bsr {

namespace {

constexpr int kTileKV = 64;    // tokens per staged KV tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int D>
struct PrefillSmem {
  static constexpr int KS = D + 8;          // K row stride (elements), +16 B against bank conflicts
  static constexpr int VS = kTileKV + 4;    // V^T row stride (elements)
  static constexpr int K_BYTES = kTileKV * KS * 2;
  static constexpr int V_BYTES = D * VS * 2;
  static constexpr int COMB_BYTES = kWaves * 16 * (D + 2) * 4;
  static constexpr int BYTES = (K_BYTES + V_BYTES) > COMB_BYTES ? (K_BYTES + V_BYTES) : COMB_BYTES;
};

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads) void attn_prefill_bf16_kernel(RunArgs a) {
  using SM = PrefillSmem<D>;
  constexpr int KB = D / 32;  // k-blocks of the score product
  constexpr int DB = D / 16;  // d-blocks of the output product
  constexpr int CH = D / 8;   // 16-byte chunks per K/V row
  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::BYTES];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vt = reinterpret_cast<uint16_t*>(smem + SM::K_BYTES);
  float* comb = reinterpret_cast<float*>(smem);

  const int w = blockIdx.x, hk = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, j = lane >> 4;
  const float c = a.sm_scale * kLog2e;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  uint16_t* __restrict__ O = static_cast<uint16_t*>(a.o);

  for (int it = a.qptr[w]; it < a.qptr[w + 1]; ++it) {
    const ItemRec item = a.items[it];
    const ReqRec rq = a.req[item.req];
    const int nrows = item.row_end - item.row_start;
    const int RB = (nrows + 15) >> 4;
    const int n_ks = RB >= 3 ? 1 : (RB == 2 ? 2 : 4);  // waves sharing a row block
    const int n_rg = kWaves / n_ks;
    const int rg = wave % n_rg, ks = wave / n_rg;
    // this wave's row blocks (at most two)
    const int rbs[2] = {rg, rg + n_rg};
    const int nrb = (rg < RB ? 1 : 0) + (n_ks == 1 && rg + n_rg < RB ? 1 : 0);

    // Q as the B operand: lane (n, j) holds row n of the block, k = kb*32 + j*8 .. +8
    bf16x8 qb[2][KB];
    int lim[2];
    int row_pos[2], row_hq[2];
    bool row_ok[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int r = item.row_start + (x < nrb ? rbs[x] : 0) * 16 + n;
      row_ok[x] = x < nrb && r < item.row_end;
      row_pos[x] = r / a.g;
      row_hq[x] = hk * a.g + r % a.g;
      lim[x] = item.kv_end;
      if (a.causal) lim[x] = min(lim[x], rq.kv_len - rq.q_len + row_pos[x] + 1);
      const uint16_t* qp = Q + (int64_t(rq.q_start + row_pos[x]) * a.Hq + row_hq[x]) * D;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok[x]) v = *reinterpret_cast<const u32x4*>(qp + kb * 32 + j * 8);
        qb[x][kb] = __builtin_bit_cast(bf16x8, v);
      }
    }

    float m[2] = {kNegInf, kNegInf}, l[2] = {0.f, 0.f};
    f32x4 oacc[2][DB];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[x][db] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int t0 = item.kv_start; t0 < item.kv_end; t0 += kTileKV) {
      __syncthreads();  // previous tile (or previous item's combine buffer) consumed
      // ---- stage the KV tile: gather rows through the page table ----
#pragma unroll
      for (int u = 0; u < (kTileKV * CH) / kThreads; ++u) {
        const int idx = tid + u * kThreads;
        const int tt = idx / CH, ch = idx % CH;
        int tok = t0 + tt;
        tok = tok < item.kv_end ? tok : item.kv_end - 1;  // clamp: masked below, never OOB
        const int64_t base = (page_row(a.indices, rq.page_start, tok, a.P, a.p_shift) * a.Hk + hk) * D + ch * 8;
        const u32x4 kv = *reinterpret_cast<const u32x4*>(K + base);
        const u32x4 vv = *reinterpret_cast<const u32x4*>(V + base);
        *reinterpret_cast<u32x4*>(Ks + tt * SM::KS + ch * 8) = kv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Vt[(ch * 8 + 2 * e) * SM::VS + tt] = uint16_t(vv[e] & 0xffffu);
          Vt[(ch * 8 + 2 * e + 1) * SM::VS + tt] = uint16_t(vv[e] >> 16);
        }
      }
      __syncthreads();

#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (x >= nrb) break;
        // scores for this wave's token blocks of the tile
        float s[4][4];
        float mt = kNegInf;
#pragma unroll
        for (int tbi = 0; tbi < 4; ++tbi) {
          const int tb = ks + tbi * n_ks;
          if (tbi * n_ks >= 4 - ks) break;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + (tb * 16 + n) * SM::KS + kb * 32 + j * 8);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[x][kb], acc, 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = t0 + tb * 16 + 4 * j + i;
            const float v = tok < lim[x] ? acc[i] * c : kNegInf;
            s[tbi][i] = v;
            mt = fmaxf(mt, v);
          }
        }
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        const float mnew = fmaxf(m[x], mt);
        const float muse = mnew == kNegInf ? 0.f : mnew;
        const float corr = exp2f(m[x] - muse);
        m[x] = mnew;
        float lsum = 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[x][db] *= corr;
#pragma unroll
        for (int tbi = 0; tbi < 4; ++tbi) {
          const int tb = ks + tbi * n_ks;
          if (tbi * n_ks >= 4 - ks) break;
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = exp2f(s[tbi][i] - muse);
            lsum += p[i];
          }
          const uint32_t p01 = pack_bf16x2(p[0], p[1]), p23 = pack_bf16x2(p[2], p[3]);
          const s16x4 pb = __builtin_bit_cast(s16x4, u32x2{p01, p23});
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const u32x2 vraw = *reinterpret_cast<const u32x2*>(Vt + (db * 16 + n) * SM::VS + tb * 16 + 4 * j);
            const s16x4 va = __builtin_bit_cast(s16x4, vraw);
            oacc[x][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, oacc[x][db], 0, 0, 0);
          }
        }
        l[x] = l[x] * corr + lsum;
      }
    }

    // row sums: each lane held the sum over its own tokens
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      l[x] += shfl_xor(l[x], 16);
      l[x] += shfl_xor(l[x], 32);
    }

    if (n_ks > 1) {
      // combine the waves that split this row block's tokens (one row block each)
      __syncthreads();
      float* mine = comb + wave * 16 * (D + 2);
      if (nrb > 0) {
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
      if (ks == 0 && nrb > 0) {
        float mm = kNegInf;
        for (int o = 0; o < n_ks; ++o) mm = fmaxf(mm, comb[(rg + o * n_rg) * 16 * (D + 2) + n * (D + 2) + D]);
        const float muse = mm == kNegInf ? 0.f : mm;
        float lt = 0.f;
        float wgt[4];
#pragma unroll
        for (int o = 0; o < 4; ++o) {
          wgt[o] = 0.f;
          if (o < n_ks) {
            const float* src = comb + (rg + o * n_rg) * 16 * (D + 2) + n * (D + 2);
            wgt[o] = exp2f(src[D] - muse);
            lt += wgt[o] * src[D + 1];
          }
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float sum = 0.f;
#pragma unroll
            for (int o = 0; o < 4; ++o)
              if (o < n_ks) sum += wgt[o] * comb[(rg + o * n_rg) * 16 * (D + 2) + n * (D + 2) + db * 16 + 4 * j + i];
            oacc[0][db][i] = sum;
          }
        m[0] = mm;
        l[0] = lt;
      }
    }

    // ---- epilogue: final output or partial state ----
    if (ks == 0) {
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (x >= nrb || !row_ok[x]) continue;
        const int r = item.row_start + rbs[x] * 16 + n;
        const bool empty = !(l[x] > 0.f);
        const float inv = empty ? 0.f : 1.f / l[x];
        const float lse = empty ? kNegInf : (m[x] + log2f(l[x])) * kLn2;
        if (item.slot < 0) {
          const int64_t orow = int64_t(rq.q_start + row_pos[x]) * a.Hq + row_hq[x];
          uint16_t* op = O + orow * D;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const f32x4 v = oacc[x][db] * inv;
            *reinterpret_cast<u32x2*>(op + db * 16 + 4 * j) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
          if (j == 0) a.lse[orow] = lse;
        } else {
          const int64_t prow = (int64_t(item.slot) * a.Hk + hk) * a.Tq + (r - item.row_start);
          float* pp = a.part_o + prow * D;
#pragma unroll
          for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(pp + db * 16 + 4 * j) = oacc[x][db] * inv;
          if (j == 0) a.part_lse[prow] = lse;
        }
      }
    }
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
