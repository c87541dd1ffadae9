// bf16 paged decode on gfx950: one query token per request, GQA-fused, split-KV.
//
// Decode reads every KV byte once and does O(g) arithmetic per byte (operational
// intensity O(g * l_qo): "FlashInfer: Engineering a Customizable, Block-Sparse
// Attention Engine for LLM Inference Serving" §II.3-II.4; eq. 2 of "FlashInfer:
// Making Attention Fit the Serving Workload"), so the kernel is built around HBM
// traffic: every wave streams the KV rows of one KV head for all G query heads of its
// group (head-group fusion, eq. 3), with one 16-byte load per lane per row chunk.
//
// Layout of a 16-token step (lane = n + 16 j, n = token within the step, j = 0..3):
//   - the lane loads K[token n][kb*32 + j*8 .. +8] and V[token n][kb*32 + j*8 .. +8]
//     for kb = 0 .. D/32-1 (page lookup per token through the BSR indices, eq. 7);
//   - S = Q_rep K^T on v_mfma_f32_16x16x32_bf16, where the 16 rows of Q_rep repeat the
//     G query heads (row r -> head r mod G): the K fragment is exactly the B operand,
//     and every lane receives the G scores of its own token n;
//   - each lane keeps its own online-softmax partial sums (l, acc) for its token
//     subsequence, sharing one running maximum per head across the wave (the step
//     maximum is a 16-lane butterfly), so rescaling happens only when the maximum
//     grows; the 16 lanes of a row are summed once at the end of the work item.
// A work item writes the final (O, LSE) or, for a split request, a partial state that
// the merge pass folds in the planned order.
#include "common.cuh"
#include "launch.h"

namespace bsr {

namespace {
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, shfl_xor(v, 1));
  v = fmaxf(v, shfl_xor(v, 2));
  v = fmaxf(v, shfl_xor(v, 4));
  v = fmaxf(v, shfl_xor(v, 8));
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += shfl_xor(v, 1);
  v += shfl_xor(v, 2);
  v += shfl_xor(v, 4);
  v += shfl_xor(v, 8);
  return v;
}
}  // namespace

// D: head dim; G: query heads handled by one wave (divides 4).
template <int D, int G>
__global__ __launch_bounds__(64) void attn_decode_bf16_kernel(RunArgs a) {
  constexpr int KB = D / 32;
  const int w = blockIdx.x;
  const int HW = a.g / G;  // waves per KV head
  const int hk = blockIdx.y / HW, hw = blockIdx.y % HW;
  const int lane = threadIdx.x, n = lane & 15, j = lane >> 4;
  const float c = a.sm_scale * kLog2e;
  const uint16_t* __restrict__ Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ K = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ V = static_cast<const uint16_t*>(a.v);
  uint16_t* __restrict__ O = static_cast<uint16_t*>(a.o);

  for (int it = a.qptr[w]; it < a.qptr[w + 1]; ++it) {
    const ItemRec item = a.items[it];
    const ReqRec rq = a.req[item.req];
    // A operand: row n of Q_rep = query head hk*g + hw*G + (n mod G)
    const int hq_row = hk * a.g + hw * G + (n % G);
    const uint16_t* qp = Q + (int64_t(rq.q_start) * a.Hq + hq_row) * D;
    bf16x8 qa[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) qa[kb] = *reinterpret_cast<const bf16x8*>(qp + kb * 32 + j * 8);

    float m[G], l[G];
    float acc[G][KB][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegInf;
      l[h] = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][kb][e] = 0.f;
    }

    for (int t0 = item.kv_start; t0 < item.kv_end; t0 += 16) {
      const int t = t0 + n;
      const bool valid = t < item.kv_end;
      const int tc = valid ? t : item.kv_end - 1;
      const int64_t base = (page_row(a.indices, rq.page_start, tc, a.P, a.p_shift) * a.Hk + hk) * D + j * 8;
      u32x4 kr[KB], vr[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        kr[kb] = *reinterpret_cast<const u32x4*>(K + base + kb * 32);
        vr[kb] = *reinterpret_cast<const u32x4*>(V + base + kb * 32);
      }
      f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kb], __builtin_bit_cast(bf16x8, kr[kb]), S, 0, 0, 0);
      // S[i] = score of query head (4j + i) mod G = i mod G for this lane's token n
      float p[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float s = valid ? S[h] * c : kNegInf;
        const float mt = row16_max(s);
        if (mt > m[h]) {  // wave-uniform: every row of the wave holds the same scores
          const float corr = exp2f(m[h] - mt);
          l[h] *= corr;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][kb][e] *= corr;
          m[h] = mt;
        }
        p[h] = exp2f(s - m[h]);
        l[h] += p[h];
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v0 = bf16_lo(vr[kb][e]), v1 = bf16_hi(vr[kb][e]);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h][kb][2 * e] += p[h] * v0;
            acc[h][kb][2 * e + 1] += p[h] * v1;
          }
        }
    }

    // sum the 16 token lanes of each row
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] = row16_sum(l[h]);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][kb][e] = row16_sum(acc[h][kb][e]);
    }

    // lane n writes the (head, kb) fragment number n; lanes j cover the 8-wide pieces
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bool empty = !(l[h] > 0.f);
      const float inv = empty ? 0.f : 1.f / l[h];
      const float lse = empty ? kNegInf : (m[h] + log2f(l[h])) * kLn2;
      const int hq = hk * a.g + hw * G + h;
      const int prow_in_tile = hw * G + h;  // packed row of a one-token request
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (n != h * KB + kb) continue;
        const int dofs = kb * 32 + j * 8;
        if (item.slot < 0) {
          uint16_t* op = O + (int64_t(rq.q_start) * a.Hq + hq) * D + dofs;
          u32x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = pack_bf16x2(acc[h][kb][2 * e] * inv, acc[h][kb][2 * e + 1] * inv);
          *reinterpret_cast<u32x4*>(op) = ov;
        } else {
          const int64_t prow = (int64_t(item.slot) * a.Hk + hk) * a.Tq + prow_in_tile;
          float* pp = a.part_o + prow * D + dofs;
          f32x4 o0, o1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o0[e] = acc[h][kb][e] * inv;
            o1[e] = acc[h][kb][4 + e] * inv;
          }
          *reinterpret_cast<f32x4*>(pp) = o0;
          *reinterpret_cast<f32x4*>(pp + 4) = o1;
        }
      }
      if (lane == 0) {
        if (item.slot < 0) a.lse[int64_t(rq.q_start) * a.Hq + hq] = lse;
        else a.part_lse[(int64_t(item.slot) * a.Hk + hk) * a.Tq + prow_in_tile] = lse;
      }
    }
  }
}

namespace {
int group_per_wave(int g) { return g <= 4 ? g : 4; }
}  // namespace

bool decode_bf16_supported(int d, int g, int Tq) {
  if (!(d == 64 || d == 128)) return false;
  if (g < 1 || g > Tq) return false;
  return g == 1 || g == 2 || g == 4 || g % 4 == 0;
}

int decode_bf16_waves_per_kv_head(int g) { return g / group_per_wave(g); }

template <int D>
static const void* decode_fn(int G) {
  switch (G) {
    case 1: return reinterpret_cast<const void*>(&attn_decode_bf16_kernel<D, 1>);
    case 2: return reinterpret_cast<const void*>(&attn_decode_bf16_kernel<D, 2>);
    default: return reinterpret_cast<const void*>(&attn_decode_bf16_kernel<D, 4>);
  }
}

int decode_bf16_blocks_per_cu(int d, int g) {
  const int G = group_per_wave(g);
  int nb = 1;
  const void* f = d == 64 ? decode_fn<64>(G) : decode_fn<128>(G);
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, f, 64, 0);
  return (e == hipSuccess && nb > 0) ? nb : 1;
}

hipError_t launch_decode_bf16(const RunArgs& a, hipStream_t s) {
  const int G = group_per_wave(a.g);
  dim3 grid(a.C, a.Hk * (a.g / G)), block(64);
#define BSR_DEC(DD, GG) hipLaunchKernelGGL((attn_decode_bf16_kernel<DD, GG>), grid, block, 0, s, a)
  if (a.d == 64) {
    if (G == 1) BSR_DEC(64, 1); else if (G == 2) BSR_DEC(64, 2); else BSR_DEC(64, 4);
  } else if (a.d == 128) {
    if (G == 1) BSR_DEC(128, 1); else if (G == 2) BSR_DEC(128, 2); else BSR_DEC(128, 4);
  } else {
    return hipErrorInvalidValue;
  }
#undef BSR_DEC
  return hipGetLastError();
}

}  // namespace bsr
