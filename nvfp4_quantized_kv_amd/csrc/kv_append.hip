// kv_quant_append and nvfp4 dequant kernels for gfx950.
//
// Append: release post of the gzenz/ninfer fork (prismix.dev), section "NVFP4
// KV cache (from scratch)", bullet 3 (the current token's K/V are quantized to
// NVFP4 in place, no separate quantization pass), with RoPE + Hadamard on K
// (bullet 2) and row-major scales (bullet 4).  One 128-element row is handled
// by 16 lanes, 8 elements each, so a wavefront quantizes 4 rows at a time; a
// lane loads its 8 inputs with one 16-byte (bf16) or two 16-byte (f32) loads
// and stores its 8 codes as one 4-byte word into the tiled code area.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4kv_codec.hpp"
#include "nvfp4kv_internal.hpp"

namespace nvfp4kv {

namespace {

// Row slots come in groups of 8: the K rows of four consecutive (token, kv
// head) pairs, then their four V rows.  The 4 rows of a wavefront are thus
// all K or all V: only K rows take RoPE and the rotation, and a wavefront
// mixing both kinds would run that path with its V lanes idle.  The rows of
// a wavefront are neighbouring input rows (1 KB of bf16 contiguous).
__global__ __launch_bounds__(256) void kv_quant_append_kernel(
    uint8_t* __restrict__ pool, int64_t num_pages, int hkv, int layer, int n_pairs,
    const void* __restrict__ k, const void* __restrict__ v, int dtype,
    const int64_t* __restrict__ slots, const int32_t* __restrict__ positions,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, int rotary_dim,
    int hadamard, SignMask signs) {
  const int lane = (int)__lane_id();
  const int r = lane & 15;
  const int row = (int)(blockIdx.x * (blockDim.x / 16) + threadIdx.x / 16);
  const int which = (row >> 2) & 1;       // 0 = K, 1 = V
  // Lanes past the last pair still take part in the shuffles, on a copy of
  // the last pair's row of their kind, and store nothing.
  int pair = (row >> 3) * 4 + (row & 3);  // token * hkv + kv head
  const bool active = pair < n_pairs;
  pair = active ? pair : n_pairs - 1;
  const int g = pair % hkv;
  const int tok = pair / hkv;
  const size_t elem_off = ((size_t)tok * hkv + g) * kHeadDim + 8 * r;
  float x[8];
  load8(which ? v : k, dtype, elem_off, x);
  const int rot = which ? 0 : rotary_dim;
  const bool had = which ? false : (hadamard != 0);
  const float* crow = nullptr;
  const float* srow = nullptr;
  if (rot > 0) {
    const int pos = positions[tok];
    crow = rope_cos + (size_t)pos * (rotary_dim / 2);
    srow = rope_sin + (size_t)pos * (rotary_dim / 2);
  }
  // K rows and V rows of a wavefront take different paths through RoPE and
  // the rotation.  Every shuffle inside reads from a lane of the same 16-lane
  // group, and all 16 lanes of a group hold the same row kind, so the source
  // lane is always active on the path that reads it.
  uint32_t codes, scode;
  quant_row16(x, r, rot, crow, srow, had, which ? 0u : lane_signs(hadamard, signs, r), codes, scode);
  if (!active) return;
  const int64_t slot = slots[tok];
  const int64_t page = slot / kPageSize;
  const uint32_t t = (uint32_t)(slot % kPageSize);
  uint8_t* blk = pool + (((size_t)layer * (size_t)num_pages + (size_t)page) * (size_t)hkv + g) *
                            (size_t)kBlockBytes;
  const uint32_t woff = which ? v_code_word_off(t, (uint32_t)r) : k_code_word_off(t, (uint32_t)r);
  *reinterpret_cast<uint32_t*>(blk + woff) = codes;
  if ((r & 1) == 0) blk[(which ? kVScaleOff : kKScaleOff) + 8 * t + r / 2] = (uint8_t)scode;
}

__device__ inline void store8(void* dst, int dtype, size_t elem_off, const float (&x)[8]) {
  if (dtype == 1) {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // the values are exact in bf16: truncation is exact
      u[i] = (__float_as_uint(x[2 * i]) >> 16) | (__float_as_uint(x[2 * i + 1]) & 0xFFFF0000u);
    }
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(dst) + elem_off) = make_uint4(u[0], u[1], u[2], u[3]);
  } else {
    float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(dst) + elem_off);
    p[0] = make_float4(x[0], x[1], x[2], x[3]);
    p[1] = make_float4(x[4], x[5], x[6], x[7]);
  }
}

__global__ __launch_bounds__(256) void nvfp4_dequant_kernel(
    const uint8_t* __restrict__ pool, int64_t num_pages, int hkv, int layer, int n_rows,
    const int64_t* __restrict__ slots, void* __restrict__ k_out, void* __restrict__ v_out,
    int dtype, int unrotate, int hadamard, SignMask signs) {
  const int r = (int)(threadIdx.x & 15);
  const int row = (int)(blockIdx.x * (blockDim.x / 16) + threadIdx.x / 16);
  const bool active = row < n_rows;
  const int rr = active ? row : n_rows - 1;
  const int which = rr & 1;
  const int g = (rr >> 1) % hkv;
  const int tok = (rr >> 1) / hkv;
  const int64_t slot = slots[tok];
  const int64_t page = slot / kPageSize;
  const uint32_t t = (uint32_t)(slot % kPageSize);
  const uint8_t* blk = pool + (((size_t)layer * (size_t)num_pages + (size_t)page) * (size_t)hkv + g) *
                                  (size_t)kBlockBytes;
  const uint32_t codes = *reinterpret_cast<const uint32_t*>(
      blk + (which ? v_code_word_off(t, (uint32_t)r) : k_code_word_off(t, (uint32_t)r)));
  const float s = e4m3_value(blk[(which ? kVScaleOff : kKScaleOff) + 8 * t + r / 2]);
  float x[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = e2m1_value((codes >> (4 * k)) & 15u) * s;
  if (unrotate && which == 0) {
    // H is symmetric and orthogonal: applying the transform again undoes it
    // (up to float rounding), and the randomized rotation's negations come
    // after it.  Every lane of the group runs the shuffles.
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k & h) continue;
        const float a = x[k], b = x[k + h];
        x[k] = a + b;
        x[k + h] = a - b;
      }
    }
#pragma unroll
    for (int bit = 1; bit < 16; bit <<= 1) {
      const bool upper = (r & bit) != 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p = __shfl_xor(x[k], bit, 64);
        x[k] = upper ? (p - x[k]) : (x[k] + p);
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = x[k] * __uint_as_float(0x3DB504F3u);
    const uint32_t neg = lane_signs(hadamard, signs, r);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if ((neg >> k) & 1u) x[k] = -x[k];
  }
  if (!active) return;
  void* dst = which ? v_out : k_out;
  if (dst == nullptr) return;
  store8(dst, dtype, ((size_t)tok * hkv + g) * kHeadDim + 8 * r, x);
}

}  // namespace

hipError_t launch_append(const LaunchPool& P, int layer, int n_tok, const void* k, const void* v,
                         int dtype, const int64_t* slots, const int32_t* positions,
                         const float* rope_cos, const float* rope_sin, hipStream_t stream) {
  const int n_pairs = n_tok * P.hkv;
  const int n_slots = 8 * ((n_pairs + 3) / 4);   // groups of 4 K rows + 4 V rows
  const int rows_per_block = 16;                 // 256 threads, 16 lanes per row
  const int grid = (n_slots + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(kv_quant_append_kernel, dim3(grid), dim3(256), 0, stream, P.base,
                     P.num_pages, P.hkv, layer, n_pairs, k, v, dtype, slots, positions, rope_cos,
                     rope_sin, P.rotary_dim, P.hadamard, P.signs);
  return hipGetLastError();
}

hipError_t launch_dequant(const LaunchPool& P, int layer, int n_tok, const int64_t* slots,
                          void* k_out, void* v_out, int dtype, int unrotate, hipStream_t stream) {
  const int n_rows = n_tok * P.hkv * 2;
  const int grid = (n_rows + 15) / 16;
  hipLaunchKernelGGL(nvfp4_dequant_kernel, dim3(grid), dim3(256), 0, stream, P.base, P.num_pages,
                     P.hkv, layer, n_rows, slots, k_out, v_out, dtype, unrotate && P.hadamard, P.hadamard,
                     P.signs);
  return hipGetLastError();
}

}  // namespace nvfp4kv
