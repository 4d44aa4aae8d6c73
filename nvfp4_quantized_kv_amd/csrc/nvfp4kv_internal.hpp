// Internal interface between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4kv {

// Bytes of one (layer, page, kv head) block: 64 tokens x (K, V) x (64 code + 8 scale bytes).
constexpr size_t kPoolBlockBytes = 9216;

struct LaunchPool {
  uint8_t* base;
  int64_t num_pages;
  int hkv;
  int rotary_dim;
  int hadamard;
};

// Split-K plan of one decode call.
struct DecodePlan {
  int pages_per_split;
  int n_splits;          // splits per (sequence, kv head)
  int group;             // query heads per kv head
};

// Workspace layout: partial accumulators [item][group][128] floats, then the
// running (max, sum) pairs [item][group] as float2; item = (seq * hkv + kvh)
// * n_splits + split.
inline size_t ws_acc_bytes(int n_seq, int hkv, const DecodePlan& pl) {
  return (size_t)n_seq * hkv * pl.n_splits * pl.group * 128 * sizeof(float);
}
inline size_t ws_bytes(int n_seq, int hkv, const DecodePlan& pl) {
  size_t a = ws_acc_bytes(n_seq, hkv, pl);
  a = (a + 255) & ~(size_t)255;
  return a + (size_t)n_seq * hkv * pl.n_splits * pl.group * 2 * sizeof(float);
}

hipError_t launch_append(const LaunchPool& P, int layer, int n_tok, const void* k, const void* v,
                         int dtype, const int64_t* slots, const int32_t* positions,
                         const float* rope_cos, const float* rope_sin, hipStream_t stream);

hipError_t launch_dequant(const LaunchPool& P, int layer, int n_tok, const int64_t* slots,
                          void* k_out, void* v_out, int dtype, int unrotate, hipStream_t stream);

hipError_t launch_decode(const LaunchPool& P, int layer, int n_seq, int n_q_heads, const void* q,
                         int q_dtype, const int32_t* q_positions, const float* rope_cos,
                         const float* rope_sin, const int32_t* page_table, int page_table_stride,
                         const int32_t* seq_lens, float sm_scale, float* out, void* workspace,
                         const DecodePlan& plan, hipStream_t stream);

}  // namespace nvfp4kv
