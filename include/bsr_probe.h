/* Measurement probes of libbsr_probe.so: the HBM read-bandwidth probe for the roofline of the
 * attention kernels, and the execution-rate probes below it.
 *
 * The attention kernels of libbsr_attn.so are priced against the 8 TB/s HBM3E peak.  What a
 * kernel can actually stream from HBM depends on the access shape: the decode path reads K and
 * V one page at a time in the order of the page table, scattered over the pool ("FlashInfer:
 * Engineering a Customizable, Block-Sparse Attention Engine for LLM Inference Serving" §V.4:
 * gathers at page granularity, contiguous inside a page).  This probe reads the same bytes in
 * the same page order and does nothing else with them, so its rate is the streaming ceiling of
 * that shape on the device it runs on.  It is a measurement tool, not part of the attention
 * path, and libbsr_attn.so does not depend on it.
 */
#ifndef BSR_PROBE_H_
#define BSR_PROBE_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read every byte of the pages `pages[0 .. n_pages)` of two pools (device memory): page p
 * occupies bytes [p * page_bytes, (p + 1) * page_bytes) of `pool_a` and of `pool_b`.  Each
 * workgroup of the grid (`grid` workgroups of 256 threads) takes pages i = blockIdx, blockIdx +
 * grid, ... and reads page pages[i] of pool_a and then of pool_b with 16-byte loads, whole
 * page per workgroup.  The loaded values are folded into one word per thread that is written
 * to `sink` (device memory, at least grid * 256 uint32_t) only if it equals a value the host
 * passes as `never` (so the loads cannot be removed); pass a value the fold cannot produce in
 * practice, or read `sink` back to check.
 *
 * Arguments: `pages` device int32 array of length n_pages, every entry in [0, pool_pages);
 * page_bytes a positive multiple of 4096; grid >= 1; `stream` a hipStream_t or NULL.
 * The caller owns every buffer.  The call only launches the kernel (asynchronous on
 * `stream`); time it with events on that stream.
 *
 * Returns 0, or -1 for invalid arguments (null pointers, n_pages < 0, page_bytes not a
 * positive multiple of 4096, grid < 1), or -2 if the launch failed.  Page ids are not
 * checked on the device: the caller guarantees them. */
int bsr_probe_read_pages(const void* pool_a, const void* pool_b, const int32_t* pages, int64_t n_pages,
                         int64_t page_bytes, int32_t grid, uint32_t never, uint32_t* sink, void* stream);

/* ---- execution-rate probes (gfx950) ----
 * Each runs a fixed instruction sequence in a loop on one or more workgroups and writes the
 * shader-clock cycles it took (s_memtime) to `cycles` (device memory).  They back the design
 * rules of the attention kernels with measurements anyone can repeat.  All return 0, -1 for
 * invalid arguments, -2 if the launch failed; they only launch (asynchronous on `stream`, a
 * hipStream_t or NULL).  `sink` (device memory) receives values derived from the loop's
 * results so that nothing is optimised away; its contents are meaningless. */

/* Modes of bsr_probe_issue_mix: one wave, 8 slots per iteration, a slot being
 *   0 one v_mfma_f32_32x32x16_bf16            4 one MFMA + four v_exp_f32
 *   1 one MFMA + six v_fma_f32                5 eight v_fma_f32 (no MFMA)
 *   2 one MFMA + eight v_fma_f32              6 eight v_exp_f32 (no MFMA)
 *   3 one MFMA + three v_exp_f32              7 one MFMA + two v_fma_f32 + two v_exp_f32
 * (accumulators rotate over four; even and odd slots use two sets of registers, so every
 * vector instruction reads a value written two slots earlier and none waits for a result).  cycles[0] = cycles of `iters` iterations (8 iters slots),
 * cycles[1] = the 100 MHz real-time counter over the same loop (for the clock).  sink: 64
 * floats. */
#define BSR_PROBE_MIX_MODES 8
int bsr_probe_issue_mix(int32_t mode, int32_t iters, uint64_t* cycles, float* sink, void* stream);

/* One workgroup of `waves` (1..4) waves, each reading the 128-row prefill kernel's LDS operand
 * pattern `iters` times: pattern 0 = eight ds_read_b128 of K fragments (1 KB each), pattern 1 =
 * sixteen ds_read_b64_tr_b16 of V (512 B each), then a wait.  cycles[w] = cycles of wave w
 * (at least `waves` entries); sink: 256 uint32_t. */
int bsr_probe_lds_read(int32_t pattern, int32_t waves, int32_t iters, uint64_t* cycles, uint32_t* sink,
                       void* stream);

/* `blocks` workgroups of `waves` (1..4) waves; every wave copies 8 KB from `src` into LDS per
 * iteration with eight 16-byte-per-lane LDS-DMA loads (global_load_lds_dwordx4) and waits for
 * them.  src: device memory of at least 32 KB (kept small so that it stays in L2).
 * cycles[4 b + w] = cycles of wave w of workgroup b (at least 4 blocks entries); sink: at least
 * blocks * 64 * waves uint32_t. */
int bsr_probe_l2_to_lds(const void* src, int32_t waves, int32_t blocks, int32_t iters, uint64_t* cycles,
                        uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif  /* BSR_PROBE_H_ */
