// HBM read-bandwidth probe (libbsr_probe.so): reads pages of two pools in a given page order,
// 16 bytes per lane per load, a whole page per workgroup.  Declared in include/bsr_probe.h.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "bsr_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kLoads = 8;  // 16-byte loads per thread in flight per batch: 32 KB per workgroup

__global__ __launch_bounds__(kThreads) void read_pages_kernel(const u32x4* __restrict__ a, const u32x4* __restrict__ b,
                                                              const int32_t* __restrict__ pages, int64_t n_pages,
                                                              int64_t page_vec, uint32_t never, uint32_t* sink) {
  uint32_t acc = 0;
  for (int64_t i = blockIdx.x; i < n_pages; i += gridDim.x) {
    const int64_t base = int64_t(pages[i]) * page_vec;
#pragma unroll
    for (int pool = 0; pool < 2; ++pool) {
      const u32x4* p = (pool == 0 ? a : b) + base;
      for (int64_t v = threadIdx.x; v < page_vec; v += kThreads * kLoads) {
        u32x4 x[kLoads];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
          const int64_t e = v + int64_t(u) * kThreads;
          x[u] = e < page_vec ? p[e] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kLoads; ++u) acc += x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
      }
    }
  }
  if (acc == never) sink[int64_t(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" int bsr_probe_read_pages(const void* pool_a, const void* pool_b, const int32_t* pages, int64_t n_pages,
                                    int64_t page_bytes, int32_t grid, uint32_t never, uint32_t* sink, void* stream) {
  if (!pool_a || !pool_b || !pages || !sink || n_pages < 0 || page_bytes <= 0 || page_bytes % 4096 != 0 || grid < 1)
    return -1;
  if (n_pages == 0) return 0;
  hipLaunchKernelGGL(read_pages_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(pool_a), static_cast<const u32x4*>(pool_b), pages, n_pages,
                     page_bytes / 16, never, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
