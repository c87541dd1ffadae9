// Probes of the gfx950 execution rates that the attention kernels are designed around
// (libbsr_probe.so, declared in include/bsr_probe.h).  Each probe runs a fixed instruction
// sequence in a loop and reports the shader-clock cycles it took (s_memtime), so that a design
// rule ("how much vector work hides under one matrix instruction", "how many bytes a CU moves
// from L2 into LDS per cycle") is a measurement anyone can repeat.  The sequences are written
// as single asm blocks that end with their own waits, so the compiler neither reorders them nor
// sees registers in flight across them.  Measurement tools only: the attention library does
// not use them.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bsr_probe.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- issue mixes: one wave, 8 slots per loop iteration ----
// A slot is at most one v_mfma_f32_32x32x16_bf16 (accumulators rotate over four, so no product
// waits for the previous one) followed by the slot's vector instructions; even slots use
// registers x0..x7 and odd slots y0..y7, so every vector instruction's input was written two
// slots earlier and none waits for a result.
#define BSR_MF(a) "v_mfma_f32_32x32x16_bf16 %[" a "], %[A], %[B], %[" a "]\n\t"
#define BSR_FM(x) "v_fma_f32 %[" x "], %[" x "], %[c], %[m]\n\t"
#define BSR_EX(x) "v_exp_f32 %[" x "], %[" x "]\n\t"
#define BSR_SLOTS8(S) S("a0", "x") S("a1", "y") S("a2", "x") S("a3", "y") S("a0", "x") S("a1", "y") S("a2", "x") S("a3", "y")
#define BSR_S_M(a, r) BSR_MF(a)
#define BSR_S_M6F(a, r) BSR_MF(a) BSR_FM(r "0") BSR_FM(r "1") BSR_FM(r "2") BSR_FM(r "3") BSR_FM(r "4") BSR_FM(r "5")
#define BSR_S_M8F(a, r) BSR_S_M6F(a, r) BSR_FM(r "6") BSR_FM(r "7")
#define BSR_S_M3E(a, r) BSR_MF(a) BSR_EX(r "0") BSR_EX(r "1") BSR_EX(r "2")
#define BSR_S_M4E(a, r) BSR_S_M3E(a, r) BSR_EX(r "3")
#define BSR_S_F8(a, r) \
  BSR_FM(r "0") BSR_FM(r "1") BSR_FM(r "2") BSR_FM(r "3") BSR_FM(r "4") BSR_FM(r "5") BSR_FM(r "6") BSR_FM(r "7")
#define BSR_S_E8(a, r) \
  BSR_EX(r "0") BSR_EX(r "1") BSR_EX(r "2") BSR_EX(r "3") BSR_EX(r "4") BSR_EX(r "5") BSR_EX(r "6") BSR_EX(r "7")
#define BSR_S_M2F2E(a, r) BSR_MF(a) BSR_FM(r "0") BSR_FM(r "1") BSR_EX(r "2") BSR_EX(r "3")
#define BSR_MIX_OPERANDS                                                                                       \
  : [a0] "+a"(a0), [a1] "+a"(a1), [a2] "+a"(a2), [a3] "+a"(a3), [x0] "+v"(x[0]), [x1] "+v"(x[1]),              \
    [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6]), [x7] "+v"(x[7]),      \
    [y0] "+v"(x[8]), [y1] "+v"(x[9]), [y2] "+v"(x[10]), [y3] "+v"(x[11]), [y4] "+v"(x[12]),                   \
    [y5] "+v"(x[13]), [y6] "+v"(x[14]), [y7] "+v"(x[15])                                                      \
  : [A] "v"(A), [B] "v"(B), [c] "v"(c), [m] "v"(m)

template <int MODE>
__global__ __launch_bounds__(64) void issue_mix_kernel(int iters, uint64_t* cycles, float* sink) {
  const int lane = threadIdx.x;
  u32x4 A, B;
  for (int i = 0; i < 4; ++i) {
    A[i] = 0x3f003f00u + uint32_t(lane);
    B[i] = 0x3f003f00u + uint32_t(i);
  }
  f32x16 a0 = {}, a1 = {}, a2 = {}, a3 = {};
  float x[16];
  for (int i = 0; i < 16; ++i) x[i] = 1e-3f * float(i + lane);
  const float c = 0.999f, m = 1e-3f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) asm volatile(BSR_SLOTS8(BSR_S_M) BSR_MIX_OPERANDS);
    if constexpr (MODE == 1) asm volatile(BSR_SLOTS8(BSR_S_M6F) BSR_MIX_OPERANDS);
    if constexpr (MODE == 2) asm volatile(BSR_SLOTS8(BSR_S_M8F) BSR_MIX_OPERANDS);
    if constexpr (MODE == 3) asm volatile(BSR_SLOTS8(BSR_S_M3E) BSR_MIX_OPERANDS);
    if constexpr (MODE == 4) asm volatile(BSR_SLOTS8(BSR_S_M4E) BSR_MIX_OPERANDS);
    if constexpr (MODE == 5) asm volatile(BSR_SLOTS8(BSR_S_F8) BSR_MIX_OPERANDS);
    if constexpr (MODE == 6) asm volatile(BSR_SLOTS8(BSR_S_E8) BSR_MIX_OPERANDS);
    if constexpr (MODE == 7) asm volatile(BSR_SLOTS8(BSR_S_M2F2E) BSR_MIX_OPERANDS);
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");  // the last products complete
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float tot = 0.f;
  for (int i = 0; i < 16; ++i) tot += x[i] + a0[i] + a1[i] + a2[i] + a3[i];
  sink[lane] = tot;
  if (lane == 0) {
    cycles[0] = t1 - t0;
    cycles[1] = r1 - r0;
  }
}

// ---- LDS reads: the 128-row prefill kernel's operand patterns ----
// pattern 0: eight ds_read_b128 of K fragments (token r32 & 15, swizzled chunk); pattern 1:
// sixteen ds_read_b64_tr_b16 of V (lane 16G + 4e + q at token 4 (G >> 1) + e, 8-byte unit
// 4 (G & 1) + q).  Every wave of the workgroup reads the same addresses; one wait per batch.
constexpr int kLdsBytes = 65536;

template <int PATTERN>
__global__ __launch_bounds__(256) void lds_read_kernel(int iters, uint64_t* cycles, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kLdsBytes / 4; i += blockDim.x) reinterpret_cast<uint32_t*>(lds)[i] = uint32_t(i) * 2654435761u;
  __syncthreads();
  const int r32 = lane & 31, h = lane >> 5, kt16 = r32 & 15, ksw = (kt16 >> 2) & 3;
  const uint32_t kaddr = uint32_t((r32 >> 4) * 4096 + 16 * (4 * kt16 + (h ^ ksw)));  // < 5.2 KB
  const int vG = lane >> 4, ve = (lane >> 2) & 3, vq = lane & 3;
  const uint32_t vaddr = 32768u + uint32_t(64 * (4 * (vG >> 1) + ve) + 8 * (4 * (vG & 1) + vq));  // < 33.3 KB
  u32x4 acc = {0u, 0u, 0u, 0u};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (PATTERN == 0) {
      u32x4 k0, k1, k2, k3, k4, k5, k6, k7;
      asm volatile(
          "ds_read_b128 %0, %8 offset:0\n\tds_read_b128 %1, %8 offset:1024\n\t"
          "ds_read_b128 %2, %8 offset:2048\n\tds_read_b128 %3, %8 offset:3072\n\t"
          "ds_read_b128 %4, %8 offset:8192\n\tds_read_b128 %5, %8 offset:9216\n\t"
          "ds_read_b128 %6, %8 offset:10240\n\tds_read_b128 %7, %8 offset:11264\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=v"(k0), "=v"(k1), "=v"(k2), "=v"(k3), "=v"(k4), "=v"(k5), "=v"(k6), "=v"(k7)
          : "v"(kaddr)
          : "memory");
      acc ^= k0 ^ k1 ^ k2 ^ k3 ^ k4 ^ k5 ^ k6 ^ k7;
    } else {
      u32x2 v[16];
      asm volatile(
          "ds_read_b64_tr_b16 %0, %16 offset:0\n\tds_read_b64_tr_b16 %1, %16 offset:512\n\t"
          "ds_read_b64_tr_b16 %2, %16 offset:1024\n\tds_read_b64_tr_b16 %3, %16 offset:1536\n\t"
          "ds_read_b64_tr_b16 %4, %16 offset:2048\n\tds_read_b64_tr_b16 %5, %16 offset:2560\n\t"
          "ds_read_b64_tr_b16 %6, %16 offset:3072\n\tds_read_b64_tr_b16 %7, %16 offset:3584\n\t"
          "ds_read_b64_tr_b16 %8, %16 offset:4096\n\tds_read_b64_tr_b16 %9, %16 offset:4608\n\t"
          "ds_read_b64_tr_b16 %10, %16 offset:5120\n\tds_read_b64_tr_b16 %11, %16 offset:5632\n\t"
          "ds_read_b64_tr_b16 %12, %16 offset:6144\n\tds_read_b64_tr_b16 %13, %16 offset:6656\n\t"
          "ds_read_b64_tr_b16 %14, %16 offset:7168\n\tds_read_b64_tr_b16 %15, %16 offset:7680\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3]), "=v"(v[4]), "=v"(v[5]), "=v"(v[6]), "=v"(v[7]),
            "=v"(v[8]), "=v"(v[9]), "=v"(v[10]), "=v"(v[11]), "=v"(v[12]), "=v"(v[13]), "=v"(v[14]), "=v"(v[15])
          : "v"(vaddr)
          : "memory");
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc[0] ^= v[i][0];
        acc[1] ^= v[i][1];
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (lane == 0) cycles[wave] = t1 - t0;
}

// ---- L2 into LDS: each wave copies 8 KB (eight 1 KB LDS-DMA loads) per iteration ----
// Wave w of a workgroup reads src bytes from 8192 w (below 8192 w + 1488) and writes LDS bytes
// [8192 w, 8192 w + 8192); it waits for its loads at the end of every iteration.
__global__ __launch_bounds__(256) void l2_to_lds_kernel(const u32x4* src, int iters, uint64_t* cycles, uint32_t* sink) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t ldsw =
      __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds)) + uint32_t(wave) * 8192u);
  const u32x4* p = src + (wave * 512 + lane);  // 16-byte units
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    // load b reads 16 bytes per lane at p + 64 b bytes (the column pieces of the prefill
    // kernel's 256-byte rows) into LDS fragment b: the instruction offset applies to the LDS
    // address as well, so M0 holds ldsw + b (1024 - 64) for offset 64 b
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:64\n\t"
        "s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:128\n\t"
        "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:192\n\t"
        "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:256\n\t"
        "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:320\n\t"
        "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:384\n\t"
        "s_mov_b32 m0, %9\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:448\n\t"
        "s_mov_b32 m0, %0\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&s"(saved)
        : "v"(p), "s"(ldsw), "s"(ldsw + 960u), "s"(ldsw + 2u * 960u), "s"(ldsw + 3u * 960u), "s"(ldsw + 4u * 960u),
          "s"(ldsw + 5u * 960u), "s"(ldsw + 6u * 960u), "s"(ldsw + 7u * 960u)
        : "memory", "scc");
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  __syncthreads();
  sink[int64_t(blockIdx.x) * blockDim.x + tid] = reinterpret_cast<const uint32_t*>(lds)[tid];
  if (lane == 0) cycles[int64_t(blockIdx.x) * 4 + wave] = t1 - t0;
}

}  // namespace

extern "C" int bsr_probe_issue_mix(int32_t mode, int32_t iters, uint64_t* cycles, float* sink, void* stream) {
  if (mode < 0 || mode >= BSR_PROBE_MIX_MODES || iters < 1 || !cycles || !sink) return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  switch (mode) {
    case 0: hipLaunchKernelGGL(issue_mix_kernel<0>, dim3(1), dim3(64), 0, s, iters, cycles, sink); break;
    case 1: hipLaunchKernelGGL(issue_mix_kernel<1>, dim3(1), dim3(64), 0, s, iters, cycles, sink); break;
    case 2: hipLaunchKernelGGL(issue_mix_kernel<2>, dim3(1), dim3(64), 0, s, iters, cycles, sink); break;
    case 3: hipLaunchKernelGGL(issue_mix_kernel<3>, dim3(1), dim3(64), 0, s, iters, cycles, sink); break;
    case 4: hipLaunchKernelGGL(issue_mix_kernel<4>, dim3(1), dim3(64), 0, s, iters, cycles, sink); break;
    case 5: hipLaunchKernelGGL(issue_mix_kernel<5>, dim3(1), dim3(64), 0, s, iters, cycles, sink); break;
    case 6: hipLaunchKernelGGL(issue_mix_kernel<6>, dim3(1), dim3(64), 0, s, iters, cycles, sink); break;
    default: hipLaunchKernelGGL(issue_mix_kernel<7>, dim3(1), dim3(64), 0, s, iters, cycles, sink); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int bsr_probe_lds_read(int32_t pattern, int32_t waves, int32_t iters, uint64_t* cycles, uint32_t* sink,
                                  void* stream) {
  if ((pattern != 0 && pattern != 1) || waves < 1 || waves > 4 || iters < 1 || !cycles || !sink) return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (pattern == 0)
    hipLaunchKernelGGL(lds_read_kernel<0>, dim3(1), dim3(64 * waves), 0, s, iters, cycles, sink);
  else
    hipLaunchKernelGGL(lds_read_kernel<1>, dim3(1), dim3(64 * waves), 0, s, iters, cycles, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int bsr_probe_l2_to_lds(const void* src, int32_t waves, int32_t blocks, int32_t iters, uint64_t* cycles,
                                   uint32_t* sink, void* stream) {
  if (!src || waves < 1 || waves > 4 || blocks < 1 || iters < 1 || !cycles || !sink) return -1;
  hipLaunchKernelGGL(l2_to_lds_kernel, dim3(blocks), dim3(64 * waves), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), iters, cycles, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
