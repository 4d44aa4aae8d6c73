// Internal interface between the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4kv {

// Bytes of one (layer, page, kv head) block: 64 tokens x (K, V) x (64 code +
// 8 scale bytes) with NVFP4 V; 64 x (64 + 8 + 256) with fp16 V.
constexpr size_t kPoolBlockBytes = 9216;
constexpr size_t kPoolBlockBytesF16V = 20992;
inline size_t pool_block_bytes(int v_format) { return v_format ? kPoolBlockBytesF16V : kPoolBlockBytes; }
// K scales' offset inside a block (the codes and the fp16 V tiles come first)
inline int pool_kscale_off(int v_format) { return v_format ? 20480 : 8192; }

// Element mask of the randomized rotation (hadamard 2): element j of a K or
// Q row is negated before the transform when bit j % 32 of word j / 32 is set.
struct SignMask {
  uint32_t w[4];
};

// Lane r's 8 bits of the mask (elements 8r .. 8r+7, bit k for element 8r+k);
// 0 unless the rotation is the randomized one.
__device__ inline uint32_t lane_signs(int hadamard, const SignMask& m, int r) {
  if (hadamard != 2) return 0u;
  const int q = r >> 2;
  const uint32_t word = q == 0 ? m.w[0] : q == 1 ? m.w[1] : q == 2 ? m.w[2] : m.w[3];
  return (word >> (8 * (r & 3))) & 0xFFu;
}

struct LaunchPool {
  uint8_t* base;
  int64_t num_pages;
  int hkv;
  int v_format;             // 0: NVFP4 V; 1: fp16 V
  int block_bytes;          // bytes of one (layer, page, kv head) block
  int ks_off;               // K scales' offset in a block
  int rotary_dim;
  int hadamard;
  SignMask signs;
  float k_scale, v_scale;   // per-tensor global scales (1 when unset)
  float k_inv, v_inv;       // their binary32 reciprocals, applied to append inputs
};

// Split-K plan of one decode call: the number of wavefronts that share the
// flattened (sequence, kv head, page) work equally.
struct DecodePlan {
  int n_waves;
  int group;             // query columns per kv head (query heads x new tokens of the launch)
};

// Partial slots: one per (segment, wave) pair that overlaps, indexed segment
// + wave, so at most n_seq * hkv + n_waves of them.
inline size_t ws_slots(int n_seq, int hkv, const DecodePlan& pl) {
  return (size_t)n_seq * hkv + (size_t)pl.n_waves;
}

// Workspace layout: partial accumulators [slot][group][128] floats, then
// (at the next 256-byte boundary) the (reference, sum) pairs [slot][group]
// as float2.
inline size_t ws_align(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t ws_acc_bytes(int n_seq, int hkv, const DecodePlan& pl) {
  return ws_slots(n_seq, hkv, pl) * pl.group * 128 * sizeof(float);
}
inline size_t ws_ml_offset(int n_seq, int hkv, const DecodePlan& pl) {
  return ws_align(ws_acc_bytes(n_seq, hkv, pl));
}
inline size_t ws_bytes(int n_seq, int hkv, const DecodePlan& pl) {
  return ws_ml_offset(n_seq, hkv, pl) + ws_slots(n_seq, hkv, pl) * pl.group * 2 * sizeof(float);
}

// Query columns per kv head that one decode launch takes: one to three
// column tiles of 16 (a plain decode step has the kv head's query heads, at
// most 16; several new tokens per sequence fill up to 48).
constexpr int kMaxDecodeColumns = 48;
inline int decode_column_tiles(int group) { return (group + 15) / 16; }

// Resident one-wavefront decode workgroups per CU for the kernels with `nt`
// column tiles, for one tile those of packed groups (up to 8 query columns)
// or the others, or the fp16-V kernel (0 if the query fails).
int decode_waves_per_cu(int nt, bool packed, bool vf16);

hipError_t launch_append(const LaunchPool& P, int layer, int n_tok, const void* k, const void* v,
                         int dtype, const int64_t* slots, const int32_t* positions,
                         const float* rope_cos, const float* rope_sin, hipStream_t stream);

// Copies whole pages (every layer and kv head) of the n_pages listed page
// ids between the pool and the arena [n_pages][num_layers][hkv][9216].
hipError_t launch_page_copy(const LaunchPool& P, int num_layers, int n_pages, const int32_t* page_ids,
                            uint8_t* arena, bool to_arena, hipStream_t stream);

// Reads every block of `layer` that a decode call over the same sequences
// reads, split over n_waves wavefronts; words[w] gets the XOR of wave w's
// 32-bit words.
hipError_t launch_stream_read(const LaunchPool& P, int layer, int n_seq, const int32_t* page_table,
                              int page_table_stride, const int32_t* seq_lens, int n_waves, uint32_t* words,
                              hipStream_t stream);

hipError_t launch_dequant(const LaunchPool& P, int layer, int n_tok, const int64_t* slots,
                          void* k_out, void* v_out, int dtype, int unrotate, hipStream_t stream);

// New query tokens of a decode call: n_qtok per sequence (1 for a plain
// decode step), this launch's columns start at token qtok0, and `heads`
// query heads share each kv head.
struct QTokens {
  int n_qtok;
  int qtok0;
  int heads;
};

hipError_t launch_decode_splits(const LaunchPool& P, int layer, int n_seq, int n_q_heads,
                                const void* q, const void* k_new, const void* v_new, int in_dtype,
                                const int32_t* q_positions, const float* rope_cos,
                                const float* rope_sin, const int32_t* page_table,
                                int page_table_stride, const int32_t* seq_lens, float sm_scale,
                                void* workspace, const DecodePlan& plan, const QTokens& qt,
                                hipStream_t stream);

// launch_decode_splits for rotary widths that are not multiples of 16
// (kernels compiled with the general rotation).
hipError_t launch_decode_splits_gr(const LaunchPool& P, int layer, int n_seq, int n_q_heads,
                                   const void* q, const void* k_new, const void* v_new, int in_dtype,
                                   const int32_t* q_positions, const float* rope_cos,
                                   const float* rope_sin, const int32_t* page_table,
                                   int page_table_stride, const int32_t* seq_lens, float sm_scale,
                                   void* workspace, const DecodePlan& plan, const QTokens& qt,
                                   hipStream_t stream);

hipError_t launch_decode_reduce(int hkv, int n_seq, int n_q_heads, const int32_t* seq_lens,
                                float* out, const void* workspace, const DecodePlan& plan,
                                const QTokens& qt, float v_scale, hipStream_t stream);

// The library's own decode workspace for callers that cannot allocate: a
// file-scope device array of kStaticWorkspaceBytes per GPU.  Returns its
// device address on the current device, looked up once per device (the
// array's name is a host-side stand-in, never a device address).
constexpr size_t kStaticWorkspaceBytes = (size_t)32 << 20;
hipError_t static_workspace(void** ptr);

}  // namespace nvfp4kv
