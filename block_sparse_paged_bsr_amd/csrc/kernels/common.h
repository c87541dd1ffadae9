// Device-side helpers shared by the attention, merge and gather kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../bsr_internal.h"

namespace bsr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Everything a run kernel needs, passed by value.
struct RunArgs {
  const ReqRec* req;
  const int32_t* indices;
  const ItemRec* items;
  const int32_t* qptr;
  const MergeRec* merge;
  const int32_t* mslots;
  const int32_t* mroff;  // partial-row offset per merge slot (records with has_roff)
  const int32_t* lpt;    // items in the plan's LPT order, as positions in `items`
  const ItemRec* items_lpt;  // copies of the items in that order; pad[0] = their merge record or -1
  int32_t* tickets;      // per workgroup group: next ticket, finished workgroups (zero between calls)
  int32_t num_items;
  const int32_t* imerge;  // per item (queue order): merge record of its split tile, or -1
  int32_t* arrive;        // [num_merge][H_kv]: partial states written (zero between calls)
  int32_t fold_in_kernel; // 1: the decode kernel folds split tiles; the merge pass writes empty tiles
  int32_t affine;         // 1: indices[x] = x (contiguous KV): page ids are computed, not loaded
  float* part_o;
  float* part_lse;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t B, Hq, Hk, g, d, P, Tq, C, causal, num_merge;
  int32_t p_shift;  // log2(page_size) when the page size is a power of two, else -1
  float sm_scale;
  int32_t window_left;  // sliding window (keys left of the diagonal), -1 = none
  float soft_cap;       // logits soft cap c (score -> c tanh(score / c)), 0 = none
  float k_scale, v_scale;  // per-tensor scales of an E4M3 KV cache (1 otherwise)
  const uint8_t* mask;     // packed custom mask (ReqRec::mask_off), or null
};

// Bit `bit` of a packed custom mask: bit b is bit b mod 8 of byte b / 8.
__device__ __forceinline__ bool mask_bit(const uint8_t* __restrict__ mask, int64_t bit) {
  return (mask[bit >> 3] >> (bit & 7)) & 1;
}

// ---- bf16 <-> fp32 ----
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f2bf_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f2bf_bits(lo) | (f2bf_bits(hi) << 16);
}

// tanh(x) = sign(x) (1 - e) / (1 + e) with e = exp(-2 |x|) in (0, 1]: one hardware exp2 and
// one reciprocal, no overflow for any |x|, absolute error a few 1e-7 (used by the soft cap)
__device__ __forceinline__ float fast_tanh(float x) {
  const float e = __builtin_amdgcn_exp2f(-2.f * kLog2e * __builtin_fabsf(x));
  return __builtin_copysignf((1.f - e) * __builtin_amdgcn_rcpf(1.f + e), x);
}

// ---- paging: physical token row of logical token t of a request (eq. 7) ----
__device__ __forceinline__ int64_t page_row(const int32_t* __restrict__ indices, int32_t page_start,
                                            int32_t t, int32_t P, int32_t p_shift) {
  int32_t pg, off;
  if (p_shift >= 0) {
    pg = t >> p_shift;
    off = t & ((1 << p_shift) - 1);
  } else {
    pg = t / P;
    off = t - pg * P;
  }
  return int64_t(indices[page_start + pg]) * P + off;
}

// ---- cross-lane helpers (wave64) ----
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

}  // namespace bsr
