// Host-side launchers of the HIP kernels (one translation unit per kernel family).
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace bsr {

// fp32 attention, one wave per packed query row (any group size, d <= 256).
bool attn_f32_supported(int d);
hipError_t launch_attn_f32(const RunArgs& a, hipStream_t s);

// bf16 tiled attention on MFMA (prefill, composable prefix level, decode fallback).
bool prefill_bf16_supported(int d, int Tq);
hipError_t launch_prefill_bf16(const RunArgs& a, hipStream_t s);
int prefill_bf16_blocks_per_cu(int d);

// bf16 paged decode: MFMA scores, GQA-fused, split-KV partials.  kv_e4m3: K and V are E4M3
// bytes with per-tensor scales (RunArgs::k_scale, v_scale); Q and O stay bf16.
bool decode_bf16_supported(int d, int g, int Tq);
// Non-causal plans whose query tiles hold at most 16 packed rows (several queries each) also run
// on the decode kernel: every row of a tile sees the same keys.
bool decode_bf16_tiles(int d, int g, int Tq);
hipError_t launch_decode_bf16(const RunArgs& a, bool kv_e4m3, hipStream_t s);
// One workgroup per worker holds min(H_kv, 8) waves, one per KV head; H_kv above 8 takes several
// workgroups per worker.
int decode_bf16_blocks_per_cu(int d, int Hk);
int decode_bf16_blocks_per_worker(int Hk);

// Reduction-map merge of partial states into final outputs (dtype of O).
hipError_t launch_merge(const RunArgs& a, int dtype, hipStream_t s);

// Elementwise (O, LSE) merge of two state arrays.
hipError_t launch_merge_state(const void* oa, const float* la, const void* ob, const float* lb,
                              void* oo, float* lo, int64_t rows, int heads, int d, int dtype,
                              hipStream_t s);

// Debug: physical row ids of every logical token.
hipError_t launch_gather_rows(const RunArgs& a, int64_t* rows, hipStream_t s);

}  // namespace bsr
