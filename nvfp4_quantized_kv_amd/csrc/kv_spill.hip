// Spill and restore of whole cache pages between the pool and an arena in
// pinned host memory (or device memory), gfx950.
//
// Release post of the gzenz/ninfer fork (prismix.dev), section "Multi-level
// prefix reuse with host-KV safety net": pages leave the GPU for a pinned
// host arena before they are evicted and come back on reuse.  A page here
// is every layer's and every kv head's block of one page id (the pool is
// [layer][page][kv head][9216 bytes]); the arena holds page i of a list at
// [i][layer][kv head][9216 bytes], so each (page, layer) is one contiguous
// run of num_kv_heads * 9216 bytes on both sides.  With a host arena the
// copy is the kernel's own loads and stores over the host link: the stores
// of a wavefront cover 1 KB runs, the loads keep many 16-byte requests in
// flight per wavefront, which is what that link needs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4kv_codec.hpp"
#include "nvfp4kv_internal.hpp"

namespace nvfp4kv {

namespace {

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// One workgroup per (list entry, layer) run, grid-strided; to_arena selects
// the direction.  Page ids outside [0, num_pages) are skipped.
__global__ __launch_bounds__(256) void page_copy_kernel(uint8_t* __restrict__ pool, int64_t num_pages,
                                                        int hkv, int num_layers,
                                                        const int32_t* __restrict__ page_ids,
                                                        int64_t n_runs, uint8_t* __restrict__ arena,
                                                        int to_arena) {
  const int64_t run_bytes = (int64_t)hkv * (int64_t)kBlockBytes;
  const int64_t vecs = run_bytes / 16;
  for (int64_t r = blockIdx.x; r < n_runs; r += gridDim.x) {
    const int64_t i = r / num_layers;
    const int layer = (int)(r - i * num_layers);
    const int64_t pid = page_ids[i];
    if (pid < 0 || pid >= num_pages) continue;
    u4* pv = reinterpret_cast<u4*>(pool + ((size_t)layer * (size_t)num_pages + (size_t)pid) * (size_t)run_bytes);
    u4* av = reinterpret_cast<u4*>(arena + (size_t)r * (size_t)run_bytes);
    if (to_arena) {
      for (int64_t v = threadIdx.x; v < vecs; v += blockDim.x) av[v] = __builtin_nontemporal_load(pv + v);
    } else {
      for (int64_t v = threadIdx.x; v < vecs; v += blockDim.x) pv[v] = av[v];
    }
  }
}

}  // namespace

hipError_t launch_page_copy(const LaunchPool& P, int num_layers, int n_pages, const int32_t* page_ids,
                            uint8_t* arena, bool to_arena, hipStream_t stream) {
  const int64_t n_runs = (int64_t)n_pages * num_layers;
  const int64_t grid = n_runs < 8192 ? n_runs : 8192;
  hipLaunchKernelGGL(page_copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream, P.base, P.num_pages,
                     P.hkv, num_layers, page_ids, n_runs, arena, to_arena ? 1 : 0);
  return hipGetLastError();
}

}  // namespace nvfp4kv
