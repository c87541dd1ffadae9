/* HBM read-bandwidth probe for the roofline of the attention kernels (libbsr_probe.so).
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

#ifdef __cplusplus
}
#endif

#endif  /* BSR_PROBE_H_ */
