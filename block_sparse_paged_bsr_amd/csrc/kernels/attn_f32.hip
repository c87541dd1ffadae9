// fp32 attention over a paged KV cache: one wave per packed (GQA-fused) query row.
//
// This is the full-precision path (fp32 storage and arithmetic).  Each workgroup is
// one persistent worker for one KV head and runs its planned queue of work items; for
// every packed row r of an item (query position floor(r / g), query head
// g * h_kv + r mod g, eq. 3 of "FlashInfer: Making Attention Fit the Serving
// Workload") it streams the item's KV chunk with the online-softmax recurrence of
// "FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine for LLM
// Inference Serving" (§II.2) and writes either the final (O, LSE) or a partial
// state for the merge pass.
// Variants ("FlashInfer 原理" §⑧; eq. 8 of the review): a sliding window raises the first
// visible key of each row, and a logits soft cap c replaces each scaled score s by
// c tanh(s / c) before the softmax; a custom mask (one bit per query and key, §VII LogitsMask)
// drops the keys whose bit is clear.
#include "common.h"
#include "launch.h"

namespace bsr {

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(RunArgs a) {
  constexpr int EPL = (D + 63) / 64;  // elements per lane
  const int w = blockIdx.x, hk = blockIdx.y, lane = threadIdx.x;
  // scores kept in log2 units; with a soft cap the dot product is taken with q sm_scale / c
  // and the score is c log2(e) tanh(.)
  const bool capped = a.soft_cap > 0.f;
  const float c = capped ? a.sm_scale / a.soft_cap : a.sm_scale * kLog2e;
  const float cap_l2 = a.soft_cap * kLog2e;
  const float* __restrict__ Q = static_cast<const float*>(a.q);
  const float* __restrict__ K = static_cast<const float*>(a.k);
  const float* __restrict__ V = static_cast<const float*>(a.v);
  float* __restrict__ O = static_cast<float*>(a.o);

  for (int it = a.qptr[w]; it < a.qptr[w + 1]; ++it) {
    const ItemRec item = a.items[it];
    const ReqRec rq = a.req[item.req];
    for (int row = item.row_start; row < item.row_end; ++row) {
      const int pos = row / a.g;
      const int hq = hk * a.g + row % a.g;
      const float* qp = Q + (int64_t(rq.q_start + pos) * a.Hq + hq) * D;
      float qv[EPL], acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int idx = lane + 64 * e;
        qv[e] = idx < D ? qp[idx] * c : 0.f;
        acc[e] = 0.f;
      }
      int kend = item.kv_end;
      if (a.causal) kend = min(kend, rq.kv_len - rq.q_len + pos + 1);
      int kbeg = item.kv_start;
      if (a.window_left >= 0) kbeg = max(kbeg, rq.kv_len - rq.q_len + pos - a.window_left);
      float m = kNegInf, l = 0.f;
      const int64_t mrow = rq.mask_off + int64_t(pos) * rq.kv_len;
      for (int t = kbeg; t < kend; ++t) {
        if (a.mask && !mask_bit(a.mask, mrow + t)) continue;
        const int64_t base = (page_row(a.indices, rq.page_start, t, a.P, a.p_shift) * a.Hk + hk) * D;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const int idx = lane + 64 * e;
          if (idx < D) s += qv[e] * K[base + idx];
        }
        s = wave_sum(s);
        if (capped) s = cap_l2 * tanhf(s);
        const float mn = fmaxf(m, s);
        const float corr = exp2f(m - mn);
        const float p = exp2f(s - mn);
        l = l * corr + p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const int idx = lane + 64 * e;
          const float vv = idx < D ? V[base + idx] : 0.f;
          acc[e] = acc[e] * corr + p * vv;
        }
        m = mn;
      }
      const bool empty = !(l > 0.f);
      const float inv = empty ? 0.f : 1.f / l;
      const float lse = empty ? kNegInf : (m + log2f(l)) * kLn2;
      if (item.slot < 0) {
        float* op = O + (int64_t(rq.q_start + pos) * a.Hq + hq) * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const int idx = lane + 64 * e;
          if (idx < D) op[idx] = acc[e] * inv;
        }
        if (lane == 0) a.lse[int64_t(rq.q_start + pos) * a.Hq + hq] = lse;
      } else {
        const int64_t prow = (int64_t(item.slot) * a.Hk + hk) * a.Tq + (row - item.row_start);
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const int idx = lane + 64 * e;
          if (idx < D) a.part_o[prow * D + idx] = acc[e] * inv;
        }
        if (lane == 0) a.part_lse[prow] = lse;
      }
    }
  }
}

bool attn_f32_supported(int d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

hipError_t launch_attn_f32(const RunArgs& a, hipStream_t s) {
  dim3 grid(a.C, a.Hk), block(64);
  switch (a.d) {
    case 16: hipLaunchKernelGGL(attn_f32_kernel<16>, grid, block, 0, s, a); break;
    case 32: hipLaunchKernelGGL(attn_f32_kernel<32>, grid, block, 0, s, a); break;
    case 64: hipLaunchKernelGGL(attn_f32_kernel<64>, grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_f32_kernel<128>, grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL(attn_f32_kernel<256>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace bsr
