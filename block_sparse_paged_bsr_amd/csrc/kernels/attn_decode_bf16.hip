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
//           as loaded, Q^T (column n = query head n mod g) is the B operand; lane (n, j)
//           receives the scores of tokens 4j..4j+3 for head n.
//   softmax per head (one column per lane group), in log2 units, with the running
//           maximum of the online-softmax recurrence ("FlashInfer: Engineering ...",
//           §II.2); the accumulator is rescaled only when the maximum grows.
//   output  O^T += V^T P^T on v_mfma_f32_16x16x16_bf16: P^T is the score accumulator
//           converted to bf16 in place (B operand), V^T comes from the step's V rows
//           staged in a wave-private LDS tile and read back with the transposing
//           LDS read of gfx950 (ds_read_b64_tr_b16, A operand).
// A work item writes the final (O, LSE) or a partial state folded by the merge pass.
// CAP: logits soft cap (eq. 8 of the review), each scaled score s becomes c tanh(s / c).  A
// sliding window needs nothing here: all rows of a decode item share one query position, so
// the planned chunks already start at the window.
#include "common.cuh"
#include "launch.h"

namespace bsr {

template <int D, bool CAP>
__global__ __launch_bounds__(64) void attn_decode_bf16_kernel(RunArgs a) {
  constexpr int KB = D / 32;  // k-blocks of the score product
  constexpr int DB = D / 16;  // d-blocks of the output product
  constexpr int VS = D + 8;   // LDS row stride (elements); 16-byte aligned rows
  __shared__ __attribute__((aligned(16))) uint16_t Vs[16 * VS];

  const int w = blockIdx.x, hk = blockIdx.y;
  const int lane = threadIdx.x, n = lane & 15, j = lane >> 4;
  const int g = a.g;
  const float c = CAP ? a.sm_scale / a.soft_cap : a.sm_scale * kLog2e;
  const float cap_l2 = a.soft_cap * kLog2e;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  uint16_t* __restrict__ O = static_cast<uint16_t*>(a.o);
  const int head_col = n < g ? n : n % g;  // query head offset served by column n

  for (int it = a.qptr[w]; it < a.qptr[w + 1]; ++it) {
    const ItemRec item = a.items[it];
    const ReqRec rq = a.req[item.req];
    const int kv_end = item.kv_end;

    // Q^T as the B operand: column n = query head hk*g + head_col
    const uint16_t* qp = Q + (int64_t(rq.q_start) * a.Hq + hk * g + head_col) * D + j * 8;
    bf16x8 qb[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qb[kb] = *reinterpret_cast<const bf16x8*>(qp + kb * 32);

    float m = kNegInf, l = 0.f;
    f32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    // page of this lane's token (lane n of a step) for the current, next and
    // next-but-one steps: the index load runs two steps ahead of the row loads
    const int pg_start = rq.page_start;
    auto page_of = [&](int t) -> int32_t {
      const int tc = min(t, kv_end - 1);
      return a.indices[pg_start + (a.p_shift >= 0 ? (tc >> a.p_shift) : tc / a.P)];
    };
    auto row_base = [&](int t, int32_t page) -> int64_t {
      const int tc = min(t, kv_end - 1);
      const int off = a.p_shift >= 0 ? (tc & ((1 << a.p_shift) - 1)) : tc - (tc / a.P) * a.P;
      return ((int64_t(page) * a.P + off) * a.Hk + hk) * D + j * 8;
    };
    int32_t pg_next = page_of(item.kv_start + 16 + n);
    u32x4 kr[KB], vr[KB];
    {
      const int64_t base = row_base(item.kv_start + n, page_of(item.kv_start + n));
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        kr[kb] = *reinterpret_cast<const u32x4*>(K + base + kb * 32);
        vr[kb] = *reinterpret_cast<const u32x4*>(V + base + kb * 32);
      }
    }

    for (int t0 = item.kv_start; t0 < kv_end; t0 += 16) {
      const bool has_next = t0 + 16 < kv_end;
      const int32_t pg_after = page_of(t0 + 32 + n);
      // request the next step's rows before touching this step's data
      u32x4 kn[KB], vn[KB];
      if (has_next) {
        const int64_t base = row_base(t0 + 16 + n, pg_next);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          kn[kb] = *reinterpret_cast<const u32x4*>(K + base + kb * 32);
          vn[kb] = *reinterpret_cast<const u32x4*>(V + base + kb * 32);
        }
      }
      pg_next = pg_after;

      // scores S^T[token 4j+i][head n]
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kb]), qb[kb], S, 0, 0, 0);

      // stage V rows (token n) for the transposing read below
      __syncthreads();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) *reinterpret_cast<u32x4*>(Vs + n * VS + kb * 32 + j * 8) = vr[kb];
      __syncthreads();

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

      if (has_next) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          kr[kb] = kn[kb];
          vr[kb] = vn[kb];
        }
      }
    }

    // lane (n, j) summed tokens 4j..4j+3 of every step; add the four token groups
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (n < g) {
      const int hq = hk * g + n;
      const bool empty = !(l > 0.f);
      const float inv = empty ? 0.f : 1.f / l;
      const float lse = empty ? kNegInf : (m + log2f(l)) * kLn2;
      if (item.slot < 0) {
        uint16_t* op = O + (int64_t(rq.q_start) * a.Hq + hq) * D + 4 * j;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const f32x4 v = oacc[db] * inv;
          *reinterpret_cast<u32x2*>(op + db * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
        if (j == 0) a.lse[int64_t(rq.q_start) * a.Hq + hq] = lse;
      } else {
        const int64_t prow = (int64_t(item.slot) * a.Hk + hk) * a.Tq + n;  // packed row = head offset
        float* pp = a.part_o + prow * D + 4 * j;
#pragma unroll
        for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(pp + db * 16) = oacc[db] * inv;
        if (j == 0) a.part_lse[prow] = lse;
      }
    }
  }
}

bool decode_bf16_supported(int d, int g, int Tq) {
  return (d == 64 || d == 128) && g >= 1 && g <= 16 && g <= Tq;
}

int decode_bf16_waves_per_kv_head(int) { return 1; }

int decode_bf16_blocks_per_cu(int d, int) {
  int nb = 1;
  hipError_t e = hipErrorInvalidValue;
  if (d == 64) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_decode_bf16_kernel<64, false>, 64, 0);
  if (d == 128) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, attn_decode_bf16_kernel<128, false>, 64, 0);
  return (e == hipSuccess && nb > 0) ? nb : 1;
}

hipError_t launch_decode_bf16(const RunArgs& a, hipStream_t s) {
  dim3 grid(a.C, a.Hk), block(64);
  const bool cap = a.soft_cap > 0.f;
  if (a.d == 64 && cap) hipLaunchKernelGGL((attn_decode_bf16_kernel<64, true>), grid, block, 0, s, a);
  else if (a.d == 64) hipLaunchKernelGGL((attn_decode_bf16_kernel<64, false>), grid, block, 0, s, a);
  else if (a.d == 128 && cap) hipLaunchKernelGGL((attn_decode_bf16_kernel<128, true>), grid, block, 0, s, a);
  else if (a.d == 128) hipLaunchKernelGGL((attn_decode_bf16_kernel<128, false>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace bsr
