// Attention-state merge kernels and the debug row gather.
//
// The merge is the reduction operator of attention states, (O, LSE) (+) (O, LSE):
// eq. 5-6 and Algorithm 1 of "FlashInfer: Making Attention Fit the Serving
// Workload" (§3.1-3.3), "FlashInfer 原理" §④.  The partial -> final reduction map of
// the plan ("FlashInfer: Engineering a Customizable, Block-Sparse Attention Engine
// for LLM Inference Serving" §VIII.5) lists, for every split query tile, its partial
// slots in KV order; each output element folds them in that fixed order with a
// shared maximum, so the result does not depend on which worker finished first
// (§VIII.3: no atomics).  Folding k states with one shared maximum m gives the same
// value as the left fold of pairwise merges in exact arithmetic: both equal
// sum_s e^(lse_s - m) O_s / sum_s e^(lse_s - m).
#include "common.h"
#include "launch.h"

namespace bsr {

namespace {

template <typename T>
__device__ __forceinline__ void store_out(T* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float v) { *p = uint16_t(f2bf_bits(v)); }

template <typename T>
__device__ __forceinline__ float load_in(const T* p);
template <>
__device__ __forceinline__ float load_in<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_in<uint16_t>(const uint16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }

}  // namespace

// One workgroup per (merge tile, chunk of kRowChunk rows, KV head), so a tile of many rows and
// many slots (a long shared prefix cut into many chunks) is merged by many workgroups.  Phase 1:
// the maximum, denominator and per-slot weights e^(lse_s - m) of every row of the chunk, with the
// tile's slot list staged in LDS and the weights kept there (kWeightSlots slots; any further
// slot's weight is recomputed from its LSE, the same expression).  Phase 2: every (row, d)
// element folds the partial outputs in slot order.  Small chunks (at most kFastSlots slots and
// two elements per thread, e.g. every split decode tile) load their partial outputs before
// phase 1, so those loads overlap the LSE reads.
constexpr int kMergeThreads = 256;
constexpr int kSlotsInLds = 1024;
constexpr int kFastSlots = 16;
constexpr int kRowChunk = 16;
constexpr int kWeightSlots = 256;

template <typename OutT>
__global__ __launch_bounds__(kMergeThreads) void merge_partials_kernel(RunArgs a, int row_chunks) {
  __shared__ int64_t s_base[kSlotsInLds];  // partial row of row 0 of this chunk, per slot
  __shared__ float s_m[kRowChunk], s_den[kRowChunk], s_w[kWeightSlots * kRowChunk];
  const int hk = blockIdx.y, tid = threadIdx.x;
  const int mi = blockIdx.x / row_chunks, r0 = (blockIdx.x % row_chunks) * kRowChunk;
  const MergeRec mr = a.merge[mi];
  if (a.fold_in_kernel && mr.slot_count > 0) return;  // folded by the attention kernel
  const int nrows = min(kRowChunk, mr.row_end - mr.row_start - r0);  // rows r0 .. r0 + nrows - 1
  if (nrows <= 0) return;  // uniform: a chunk past the tile's last row
  const int ns = mr.slot_count;
  const int D = a.d;
  const int* __restrict__ slots = a.mslots + mr.slot_begin;
  const int* __restrict__ roffs = a.mroff + mr.slot_begin;
  const bool has_roff = mr.has_roff != 0;
  const bool cached = ns <= kSlotsInLds;
  auto base_of = [&](int k) -> int64_t {
    return (int64_t(slots[k]) * a.Hk + hk) * a.Tq + (has_roff ? roffs[k] : 0) + r0;
  };
  if (cached)
    for (int k = tid; k < ns; k += kMergeThreads) s_base[k] = base_of(k);
  __syncthreads();
  // partial-state row of the k-th slot of the list for row r of this chunk (one LDS read per
  // slot, so the unrolled folds below issue their loads together)
  auto prow_at = [&](int k, int r) { return (cached ? s_base[k] : base_of(k)) + r; };

  const bool fast = ns <= kFastSlots && nrows * D <= 2 * kMergeThreads;  // uniform
  float ov[2][kFastSlots];
  if (fast) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * kMergeThreads;
      const int lr = idx / D, e = idx - lr * D;
#pragma unroll
      for (int k = 0; k < kFastSlots; ++k) {
        ov[u][k] = 0.f;
        if (idx < nrows * D && k < ns) ov[u][k] = a.part_o[prow_at(k, lr) * D + e];
      }
    }
  }

  // phase 1: tpr lanes of one wave per row
  int rp2 = 1;
  while (rp2 < nrows) rp2 <<= 1;
  const int tpr = min(64, kMergeThreads / rp2);
  const int r = tid / tpr, sub = tid % tpr;
  float mx = kNegInf;
  if (r < nrows)
    for (int k = sub; k < ns; k += tpr) mx = fmaxf(mx, a.part_lse[prow_at(k, r)]);
  for (int o = 1; o < tpr; o <<= 1) mx = fmaxf(mx, shfl_xor(mx, o));
  float den = 0.f;
  if (r < nrows && mx != kNegInf)
    for (int k = sub; k < ns; k += tpr) {
      const float l = a.part_lse[prow_at(k, r)];
      const float w = l == kNegInf ? 0.f : expf(l - mx);
      den += w;
      if (k < kWeightSlots) s_w[k * kRowChunk + r] = w;
    }
  for (int o = 1; o < tpr; o <<= 1) den += shfl_xor(den, o);
  if (r < nrows && sub == 0) {
    s_m[r] = mx;
    s_den[r] = den;
  }
  __syncthreads();

  // phase 2: weighted sum of the partial outputs, slot order fixed by the plan
  OutT* O = static_cast<OutT*>(a.o);
  auto finish = [&](int lr, int e, float acc) {
    const float m = s_m[lr];
    const int row = mr.row_start + r0 + lr;
    const int64_t orow = int64_t(mr.q_start + row / a.g) * a.Hq + hk * a.g + row % a.g;
    store_out<OutT>(O + orow * D + e, m == kNegInf ? 0.f : acc / s_den[lr]);
    if (e == 0) a.lse[orow] = m == kNegInf ? kNegInf : m + logf(s_den[lr]);
  };
  if (fast) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = tid + u * kMergeThreads;
      if (idx >= nrows * D) continue;
      const int lr = idx / D, e = idx - lr * D;
      const float m = s_m[lr];
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < kFastSlots; ++k)
        if (k < ns && m != kNegInf) acc += s_w[k * kRowChunk + lr] * ov[u][k];
      finish(lr, e, acc);
    }
    return;
  }
  for (int idx = tid; idx < nrows * D; idx += kMergeThreads) {
    const int lr = idx / D, e = idx - lr * D;
    const float m = s_m[lr];
    float acc = 0.f;
    if (m != kNegInf) {
      const int nw = min(ns, kWeightSlots);
      // unrolled by the slot count (uniform), so that the loads of a short fold are issued together;
      // the slots' row bases come from LDS (a slot list beyond it takes the plain loop)
      auto fold = [&](int k) { acc += s_w[k * kRowChunk + lr] * a.part_o[(s_base[k] + lr) * D + e]; };
      if (!cached) {
        for (int k = 0; k < nw; ++k) acc += s_w[k * kRowChunk + lr] * a.part_o[prow_at(k, lr) * D + e];
      } else if (nw >= 8) {
#pragma unroll 8
        for (int k = 0; k < nw; ++k) fold(k);
      } else if (nw >= 4) {
#pragma unroll 4
        for (int k = 0; k < nw; ++k) fold(k);
      } else {
#pragma unroll 2
        for (int k = 0; k < nw; ++k) fold(k);
      }
      for (int k = nw; k < ns; ++k) {
        const int64_t prow = prow_at(k, lr);
        const float l = a.part_lse[prow];
        acc += (l == kNegInf ? 0.f : expf(l - m)) * a.part_o[prow * D + e];
      }
    }
    finish(lr, e, acc);
  }
}

// Elementwise merge of two state arrays.  A 16-lane group owns one (row, head) state,
// reads both LSEs before any store, and so tolerates o_out/lse_out aliasing an input.
template <typename T>
__global__ __launch_bounds__(256) void merge_state_kernel(const T* oa, const float* la, const T* ob,
                                                         const float* lb, T* oo, float* lo,
                                                         int64_t nstates, int D) {
  const int64_t st = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  if (st >= nstates) return;
  const float a_l = la[st], b_l = lb[st];
  const bool va = a_l != kNegInf, vb = b_l != kNegInf;
  const float mx = fmaxf(a_l, b_l);
  const float wa = va ? expf(a_l - mx) : 0.f;
  const float wb = vb ? expf(b_l - mx) : 0.f;
  const float den = wa + wb;
  for (int e = sub; e < D; e += 16) {
    const float xa = va ? load_in<T>(oa + st * D + e) : 0.f;
    const float xb = vb ? load_in<T>(ob + st * D + e) : 0.f;
    float r;
    if (va && vb) r = (wa * xa + wb * xb) / den;
    else if (va) r = xa;
    else if (vb) r = xb;
    else r = 0.f;
    store_out<T>(oo + st * D + e, r);
  }
  if (sub == 0) lo[st] = (va || vb) ? mx + logf(den) : kNegInf;
}

// Physical row of every logical token, with the attention kernels' address function.
__global__ __launch_bounds__(256) void gather_rows_kernel(RunArgs a, int64_t* rows) {
  const ReqRec rq = a.req[blockIdx.x];
  for (int t = threadIdx.x; t < rq.kv_len; t += blockDim.x)
    rows[int64_t(rq.tok_start) + t] = page_row(a.indices, rq.page_start, t, a.P, a.p_shift);
}

hipError_t launch_merge(const RunArgs& a, int dtype, hipStream_t s) {
  if (a.num_merge == 0) return hipSuccess;
  const int row_chunks = (a.Tq + kRowChunk - 1) / kRowChunk;
  if (int64_t(a.num_merge) * row_chunks > INT32_MAX) return hipErrorInvalidConfiguration;
  dim3 grid(a.num_merge * row_chunks, a.Hk), block(kMergeThreads);
  if (dtype == BSR_DTYPE_F32) hipLaunchKernelGGL(merge_partials_kernel<float>, grid, block, 0, s, a, row_chunks);
  else hipLaunchKernelGGL(merge_partials_kernel<uint16_t>, grid, block, 0, s, a, row_chunks);
  return hipGetLastError();
}

hipError_t launch_merge_state(const void* oa, const float* la, const void* ob, const float* lb,
                              void* oo, float* lo, int64_t rows, int heads, int d, int dtype,
                              hipStream_t s) {
  const int64_t nst = rows * heads;
  if (nst == 0) return hipSuccess;
  const int64_t blocks = (nst * 16 + 255) / 256;
  if (dtype == BSR_DTYPE_F32)
    hipLaunchKernelGGL(merge_state_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const float*>(oa), la, static_cast<const float*>(ob), lb,
                       static_cast<float*>(oo), lo, nst, d);
  else
    hipLaunchKernelGGL(merge_state_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(oa), la, static_cast<const uint16_t*>(ob), lb,
                       static_cast<uint16_t*>(oo), lo, nst, d);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const RunArgs& a, int64_t* rows, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(a.B), dim3(256), 0, s, a, rows);
  return hipGetLastError();
}

}  // namespace bsr
