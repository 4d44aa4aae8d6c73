// Spill and restore of whole cache pages between the pool and an arena in
// pinned host memory (or device memory), gfx950.
//
// Release post of the gzenz/ninfer fork (prismix.dev), section "Multi-level
// prefix reuse with host-KV safety net": pages leave the GPU for a pinned
// host arena before they are evicted and come back on reuse.  A page here
// is every layer's and every kv head's block of one page id (the pool is
// [layer][page][kv head][block], a block 9216 bytes, or 20992 when V is kept
// in fp16); the arena holds page i of a list at [i][layer][kv head][block],
// so each (page, layer) is one contiguous run of num_kv_heads blocks on both
// sides.  With a host arena the
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
                                                        int hkv, int num_layers, int block_bytes,
                                                        const int32_t* __restrict__ page_ids,
                                                        int64_t n_runs, uint8_t* __restrict__ arena,
                                                        int to_arena) {
  const int64_t run_bytes = (int64_t)hkv * (int64_t)block_bytes;   // a multiple of 16
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

// Read-bandwidth probe of the decode kernel's access pattern: wave w reads
// the 9216-byte blocks of flat pages [w*TP/W, (w+1)*TP/W) of `layer` (the
// pages of segment seq * hkv + kvh in order, the segments in order), nine
// 16-byte non-temporal loads per lane and block, the next block's loads in
// flight while the current one is folded, and writes the XOR of the 32-bit
// words it read to words[w].
__global__ __launch_bounds__(64) void stream_read_kernel(const uint8_t* __restrict__ pool, int64_t num_pages,
                                                         int hkv, int layer, int n_seq,
                                                         const int32_t* __restrict__ page_table, int pt_stride,
                                                         const int32_t* __restrict__ seq_lens,
                                                         uint32_t* __restrict__ words) {
  const int lane = (int)threadIdx.x;
  const int64_t W = gridDim.x, w = blockIdx.x;
  auto pages_of = [&](int s) { return (int64_t)((seq_lens[s] + kPageSize - 1) / kPageSize); };
  int64_t TP = 0;
  for (int s = 0; s < n_seq; ++s) TP += pages_of(s);
  TP *= hkv;
  const int64_t x0 = (w * TP) / W, x1 = ((w + 1) * TP) / W;
  // position of flat page x0: sequence, kv head, page of the segment
  int seq = 0, kvh = 0;
  int64_t j = x0;
  while (seq < n_seq && j >= hkv * pages_of(seq)) {
    j -= hkv * pages_of(seq);
    ++seq;
  }
  if (seq < n_seq) {
    kvh = (int)(j / pages_of(seq));
    j -= kvh * pages_of(seq);
  }
  const uint8_t* layer_base = pool + (size_t)layer * (size_t)num_pages * (size_t)hkv * (size_t)kBlockBytes;
  auto block = [&](int sq, int kv, int64_t pg) {
    const int page = page_table[(size_t)sq * pt_stride + pg];
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(layer_base + ((size_t)page * hkv + kv) * (size_t)kBlockBytes), 0, kBlockBytes,
        0x00020000);
  };
  auto advance = [&](int& sq, int& kv, int64_t& pg) {
    if (++pg == pages_of(sq)) {
      pg = 0;
      if (++kv == hkv) {
        kv = 0;
        do { ++sq; } while (sq < n_seq && pages_of(sq) == 0);
      }
    }
  };
  u4 acc = {0u, 0u, 0u, 0u};
  u4 cur[9], nxt[9];
  const int voff = 16 * lane;
  if (x0 < x1) {
    const __amdgpu_buffer_rsrc_t r = block(seq, kvh, j);
#pragma unroll
    for (int i = 0; i < 9; ++i)
      cur[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 1024 * i, 2));
  }
  for (int64_t x = x0; x < x1; ++x) {
    int sq = seq, kv = kvh;
    int64_t pg = j;
    advance(sq, kv, pg);
    const bool more = x + 1 < x1;
    const __amdgpu_buffer_rsrc_t r = more ? block(sq, kv, pg)
                                          : __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(pool), 0, 0,
                                                                              0x00020000);
#pragma unroll
    for (int i = 0; i < 9; ++i)
      nxt[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 1024 * i, 2));
#pragma unroll
    for (int i = 0; i < 9; ++i) acc ^= cur[i];
#pragma unroll
    for (int i = 0; i < 9; ++i) cur[i] = nxt[i];
    seq = sq;
    kvh = kv;
    j = pg;
  }
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) v ^= (uint32_t)__shfl_xor((int)v, o, 64);
  if (lane == 0) words[w] = v;
}

}  // namespace

hipError_t launch_stream_read(const LaunchPool& P, int layer, int n_seq, const int32_t* page_table,
                              int page_table_stride, const int32_t* seq_lens, int n_waves, uint32_t* words,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)n_waves), dim3(64), 0, stream, P.base, P.num_pages,
                     P.hkv, layer, n_seq, page_table, page_table_stride, seq_lens, words);
  return hipGetLastError();
}

hipError_t launch_page_copy(const LaunchPool& P, int num_layers, int n_pages, const int32_t* page_ids,
                            uint8_t* arena, bool to_arena, hipStream_t stream) {
  const int64_t n_runs = (int64_t)n_pages * num_layers;
  const int64_t grid = n_runs < 8192 ? n_runs : 8192;
  hipLaunchKernelGGL(page_copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream, P.base, P.num_pages,
                     P.hkv, num_layers, P.block_bytes, page_ids, n_runs, arena, to_arena ? 1 : 0);
  return hipGetLastError();
}

}  // namespace nvfp4kv
