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

// x from lane r ^ BIT of the same 16-lane row (BIT = 1, 2, 4 or 8), through
// DPP: quad permutes for 1 and 2; for 4 the half-row mirror (r ^ 7) then the
// quad reversal (^ 3); for 8 the row mirror (r ^ 15) then the half-row mirror.
// Every lane has a source lane in these patterns, so bound_ctrl is set: the
// compiler then needs no copy of the `old` operand (and no wait states for
// it) before each move.
template <int BIT>
__device__ __forceinline__ float xor_lane(float x) {
  const int i = __float_as_int(x);
  int o;
  if (BIT == 1) {
    o = __builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, true);
  } else if (BIT == 2) {
    o = __builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, true);
  } else if (BIT == 4) {
    o = __builtin_amdgcn_update_dpp(0, __builtin_amdgcn_update_dpp(0, i, 0x141, 0xF, 0xF, true), 0x1B, 0xF,
                                    0xF, true);
  } else {
    o = __builtin_amdgcn_update_dpp(0, __builtin_amdgcn_update_dpp(0, i, 0x140, 0xF, 0xF, true), 0x141, 0xF,
                                    0xF, true);
  }
  return __int_as_float(o);
}

// One cross-lane stage of the transform: the lower lane of a pair keeps
// a + b, the upper one b - a (its own value subtracted from the partner's),
// as one fused multiply-add by +-1, which rounds exactly as the addition or
// subtraction does.
template <int BIT>
__device__ __forceinline__ void fwht_stage(float (&x)[8], int r) {
  const float sgn = (r & BIT) ? -1.0f : 1.0f;
  if (BIT >= 4) {
    // two chained row permutes: the first for all 8 elements, then the
    // second, so no permute waits on the one just before it
    const int c1 = BIT == 4 ? 0x141 : 0x140, c2 = BIT == 4 ? 0x1B : 0x141;
    int t[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) t[k] = __builtin_amdgcn_update_dpp(0, __float_as_int(x[k]), c1, 0xF, 0xF, true);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      x[k] = __builtin_fmaf(sgn, x[k], __int_as_float(__builtin_amdgcn_update_dpp(0, t[k], c2, 0xF, 0xF, true)));
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = __builtin_fmaf(sgn, x[k], xor_lane<BIT>(x[k]));
  }
}

// E2M1 magnitude code of |y| for block scale s by a three-level search over
// the same exact thresholds as e2m1_code: 1.75s (>=) splits codes 0-3 from
// 4-7, then 0.75s or 3.5s (>=), then 0.25s, 1.25s, 2.5s or 5s (>).  The
// thresholds increase and each test is monotone in |y|, so the result is the
// count of thresholds passed, as in e2m1_code.
__device__ __forceinline__ uint32_t e2m1_code_search(float y, const float (&t)[7], float s) {
  const float a = fabsf(y);
  const bool b2 = a >= t[3];
  const bool b1 = a >= (b2 ? t[5] : t[1]);
  const float t0 = b2 ? (b1 ? t[6] : t[4]) : (b1 ? t[2] : t[0]);
  const bool b0 = a > t0;
  uint32_t c = (b2 ? 4u : 0u) | (b1 ? 2u : 0u) | (b0 ? 1u : 0u);
  if (s == 0.0f) c = 0;
  return c | (signbit(y) ? 8u : 0u);
}

// RoPE coefficients of lane r of a row (16 lanes, 8 elements each) at one
// position: 16-byte vector reads of the table rows; lanes outside the
// rotary dims read the first entries and do not use them.
struct RopeLane {
  float cv[8], sv[8];
  bool first, in_rot;
  int src;   // the lane of the row holding the partner elements
};

// GR (rotary widths that are not a multiple of 16): coefficients element by
// element (rope_coeffs), the rotation by rope_rows_any.  The general code is
// only in the GR instances of the kernel.
template <bool GR>
__device__ __forceinline__ void rope_lane(int r, int rotary_dim, const float* cos_row, const float* sin_row,
                                          RopeLane& rl) {
  if (GR && (rotary_dim & 15) != 0) {
    rope_coeffs<true>(r, rotary_dim, cos_row, sin_row, rl.cv, rl.sv);
    rl.first = rl.in_rot = false;
    rl.src = r;
    return;
  }
  const int half = rotary_dim / 2;          // a multiple of 8
  const int hl = half / 8;                  // lanes per half
  rl.first = r < hl;
  rl.in_rot = r < 2 * hl;
  const int base = rl.in_rot ? (rl.first ? 8 * r : 8 * r - half) : 0;
  const float4* cp = reinterpret_cast<const float4*>(cos_row + base);
  const float4* sp = reinterpret_cast<const float4*>(sin_row + base);
  const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
  rl.cv[0] = c0.x; rl.cv[1] = c0.y; rl.cv[2] = c0.z; rl.cv[3] = c0.w;
  rl.cv[4] = c1.x; rl.cv[5] = c1.y; rl.cv[6] = c1.z; rl.cv[7] = c1.w;
  rl.sv[0] = s0.x; rl.sv[1] = s0.y; rl.sv[2] = s0.z; rl.sv[3] = s0.w;
  rl.sv[4] = s1.x; rl.sv[5] = s1.y; rl.sv[6] = s1.z; rl.sv[7] = s1.w;
  rl.src = rl.in_rot ? (rl.first ? r + hl : r - hl) : r;
}

// The append kernel's row quantizer: what quant_row16 computes, bit for bit
// (same binary32 operations in the same order), with the RoPE coefficients
// read beforehand (`rl`, used when `rope`), RoPE without branches, the
// transform's cross-lane stages through DPP and the E2M1 code by search.
// All 16 lanes of a row must call it together.
template <bool GR>
__device__ __forceinline__ void append_row16(float (&x)[8], int r, bool rope, int rotary_dim,
                                             const RopeLane& rl, bool hadamard, uint32_t neg, uint32_t& codes,
                                             uint32_t& scode) {
#pragma clang fp contract(off)
  const int lane = (int)__lane_id();
  if (GR && rope && (rotary_dim & 15) != 0) {
    rope_rows_any(x, r, rotary_dim / 2, rl.cv, rl.sv);
  } else if (rope) {
    const int src_lane = (lane & ~15) + rl.src;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float other = __shfl(x[k], src_lane, 64);
      // first half: x c - o s; second half: x c + o s (a - b is a + (-b))
      const float t = x[k] * rl.cv[k] + other * (rl.first ? -rl.sv[k] : rl.sv[k]);
      x[k] = rl.in_rot ? t : x[k];
    }
  }
  if (hadamard) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if ((neg >> k) & 1u) x[k] = -x[k];
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
    fwht_stage<1>(x, r);
    fwht_stage<2>(x, r);
    fwht_stage<4>(x, r);
    fwht_stage<8>(x, r);
    const float inv_sqrt128 = __uint_as_float(0x3DB504F3u);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = x[k] * inv_sqrt128;
  }
  float am = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(x[k]));
  am = fmaxf(am, xor_lane<1>(am));
  scode = e4m3_scale_code(am);
  const float s = e4m3_value(scode);
  const float t[7] = {0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.0f * s};
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) w |= e2m1_code_search(x[k], t, s) << (4 * k);
  codes = w;
}

// A lane's 8 inputs of a row as raw words: bf16 (DT 1) takes 4 words, f32
// (DT 0) 8.
template <int DT>
struct RawRow {
  uint32_t w[DT == 1 ? 4 : 8];
};

template <int DT>
__device__ __forceinline__ void load_raw(const void* src, size_t elem_off, RawRow<DT>& rw) {
  if (DT == 1) {
    const uint4 q = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(src) + elem_off);
    rw.w[0] = q.x; rw.w[1] = q.y; rw.w[2] = q.z; rw.w[3] = q.w;
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(src) + elem_off);
    const uint4 a = p[0], b = p[1];
    rw.w[0] = a.x; rw.w[1] = a.y; rw.w[2] = a.z; rw.w[3] = a.w;
    rw.w[4] = b.x; rw.w[5] = b.y; rw.w[6] = b.z; rw.w[7] = b.w;
  }
}

template <int DT>
__device__ __forceinline__ void raw_to_float(const RawRow<DT>& rw, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < (DT == 1 ? 4 : 8); ++i) {
    if (DT == 1) {
      x[2 * i] = __uint_as_float(rw.w[i] << 16);
      x[2 * i + 1] = __uint_as_float(rw.w[i] & 0xFFFF0000u);
    } else {
      x[i] = __uint_as_float(rw.w[i]);
    }
  }
}

// One workgroup (8 wavefronts) per run of 64 consecutive tokens, every kv
// head in turn, in passes of 16 tokens: wavefronts 0-3 take the 16 tokens' K
// rows, 4-7 their V rows (4 rows of 16 lanes each), so every wavefront's rows
// are all K or all V and only K rows run RoPE and the rotation.  The kv heads
// of a token share its RoPE table rows, read once into the CU's L2.
// Software pipeline over a wavefront's rows: an iteration first issues the
// loads of its own RoPE coefficients, then those of the next row (its
// token's slot and position and the row itself, unconditionally, with the
// indices clamped), then quantizes its row; so a row's chain of dependent
// loads (position, then table) overlaps the quantization of the row before
// (one row per chain and nothing in flight meanwhile made the kernel bound
// by load latency).  Consecutive tokens of a prefill sit in consecutive
// slots, whose code bytes share 128-byte lines (16 bytes per token in the K
// tiles, 4 in the V tiles) and whose scale bytes do too: one workgroup
// completes those lines in its CU's L2.  Spread over workgroups (and so over
// XCDs), each line was written back in pieces: twice the algorithmic write
// traffic, measured.
template <int DT, bool GR>
__global__ __launch_bounds__(512) void kv_quant_append_kernel(
    uint8_t* __restrict__ pool, int64_t num_pages, int hkv, int layer, int n_tok,
    const void* __restrict__ k, const void* __restrict__ v,
    const int64_t* __restrict__ slots, const int32_t* __restrict__ positions,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, int rotary_dim,
    int hadamard, SignMask signs, float k_inv, float v_inv, int v_format, int block_bytes, int ks_off) {
  const int lane = (int)__lane_id();
  const int r = lane & 15;
  const int wv = (int)(threadIdx.x >> 6);
  const int which = wv >> 2;                       // 0 = K, 1 = V
  const bool vf16 = which && v_format;             // V rows kept in fp16 (uniform per wavefront)
  const int rot = which ? 0 : rotary_dim;
  const bool had = which ? false : (hadamard != 0);
  const uint32_t neg = which ? 0u : lane_signs(hadamard, signs, r);
  const void* src = which ? v : k;
  const float inv = which ? v_inv : k_inv;   // 1 / the global scale
  const int n_it = 4 * hkv;
  // token of iteration `it` (kv head it % hkv, pass it / hkv); lanes past
  // the last token take a copy of the last token's row of their kind (they
  // still take part in the shuffles) and store nothing
  auto token = [&](int it) {
    return min((int)blockIdx.x * 64 + (it / hkv) * 16 + (wv & 3) * 4 + (lane >> 4), n_tok - 1);
  };
  // the next row's inputs, loaded one iteration ahead
  auto fetch = [&](int it, int64_t& slot, int& pos, RawRow<DT>& rw) {
    it = min(it, n_it - 1);
    const int tok = token(it);
    slot = slots[tok];
    pos = rot > 0 ? positions[tok] : 0;
    load_raw<DT>(src, ((size_t)tok * hkv + it % hkv) * kHeadDim + 8 * r, rw);
  };
  int64_t slot;
  int pos;
  RawRow<DT> rw;
  fetch(0, slot, pos, rw);
#pragma unroll 1
  for (int it = 0; it < n_it; ++it) {
    const int g = it % hkv;
    const bool active = (int)blockIdx.x * 64 + (it / hkv) * 16 + (wv & 3) * 4 + (lane >> 4) < n_tok;
    RopeLane rl;
    if (rot > 0)
      rope_lane<GR>(r, rotary_dim, rope_cos + (size_t)pos * (rotary_dim / 2),
                    rope_sin + (size_t)pos * (rotary_dim / 2), rl);
    __builtin_amdgcn_sched_barrier(0);
    int64_t slot_n;
    int pos_n;
    RawRow<DT> rw_n;
    fetch(it + 1, slot_n, pos_n, rw_n);
    __builtin_amdgcn_sched_barrier(0);
    float x[8];
    raw_to_float<DT>(rw, x);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] *= inv;
    const int64_t page = slot / kPageSize;
    const uint32_t t = (uint32_t)(slot % kPageSize);
    uint8_t* blk = pool + (((size_t)layer * (size_t)num_pages + (size_t)page) * (size_t)hkv + g) *
                              (size_t)block_bytes;
    if (vf16) {
      // V kept in fp16: element 8r + k rounded to nearest even, into its tile
      if (active) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
          *reinterpret_cast<uint16_t*>(blk + v16_off(t, (uint32_t)(8 * r + k))) = (uint16_t)f16_bits(x[k]);
      }
    } else {
      uint32_t codes, scode;
      append_row16<GR>(x, r, rot > 0, rot, rl, had, neg, codes, scode);
      if (active) {
        const uint32_t woff = which ? v_code_word_off(t, (uint32_t)r) : k_code_word_off(t, (uint32_t)r);
        *reinterpret_cast<uint32_t*>(blk + woff) = codes;
        if ((r & 1) == 0) blk[(which ? kVScaleOff : ks_off) + 8 * t + r / 2] = (uint8_t)scode;
      }
    }
    slot = slot_n;
    pos = pos_n;
    rw = rw_n;
  }
}

__device__ inline void store8(void* dst, int dtype, size_t elem_off, const float (&x)[8]) {
  if (dtype == 1) {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // bf16 nearest with ties to even (exact for the NVFP4 block values,
      // which have at most 6 significant bits; fp16 V values and un-rotated
      // rows are rounded)
      uint32_t a = __float_as_uint(x[2 * i]), b = __float_as_uint(x[2 * i + 1]);
      a = (a + 0x7FFFu + ((a >> 16) & 1u)) >> 16;
      b = (b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u;
      u[i] = a | b;
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
    int dtype, int unrotate, int hadamard, SignMask signs, float k_scale, float v_scale, int v_format,
    int block_bytes, int ks_off) {
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
                                  (size_t)block_bytes;
  float x[8];
  if (which && v_format) {
    // fp16 V: the stored values, exactly
#pragma unroll
    for (int k = 0; k < 8; ++k)
      x[k] = (float)__builtin_bit_cast(_Float16, *reinterpret_cast<const uint16_t*>(blk + v16_off(t, (uint32_t)(8 * r + k))));
  } else {
    const uint32_t codes = *reinterpret_cast<const uint32_t*>(
        blk + (which ? v_code_word_off(t, (uint32_t)r) : k_code_word_off(t, (uint32_t)r)));
    const float s = e4m3_value(blk[(which ? kVScaleOff : ks_off) + 8 * t + r / 2]);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = e2m1_value((codes >> (4 * k)) & 15u) * s;
  }
  // times the global scale (binary32 product of the exact block value)
  const float gs = which ? v_scale : k_scale;
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = x[k] * gs;
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
  const int runs = (n_tok + 63) / 64;            // 64 tokens, every kv head, per workgroup
  // the general rotation only in the kernels of widths that need it
  const bool gr = (P.rotary_dim & 15) != 0;
  auto kern = dtype == 1 ? (gr ? kv_quant_append_kernel<1, true> : kv_quant_append_kernel<1, false>)
                         : (gr ? kv_quant_append_kernel<0, true> : kv_quant_append_kernel<0, false>);
  hipLaunchKernelGGL(kern, dim3(runs), dim3(512), 0, stream, P.base, P.num_pages, P.hkv, layer, n_tok, k,
                     v, slots, positions, rope_cos, rope_sin, P.rotary_dim, P.hadamard, P.signs, P.k_inv,
                     P.v_inv, P.v_format, P.block_bytes, P.ks_off);
  return hipGetLastError();
}

hipError_t launch_dequant(const LaunchPool& P, int layer, int n_tok, const int64_t* slots,
                          void* k_out, void* v_out, int dtype, int unrotate, hipStream_t stream) {
  const int n_rows = n_tok * P.hkv * 2;
  const int grid = (n_rows + 15) / 16;
  hipLaunchKernelGGL(nvfp4_dequant_kernel, dim3(grid), dim3(256), 0, stream, P.base, P.num_pages,
                     P.hkv, layer, n_rows, slots, k_out, v_out, dtype, unrotate && P.hadamard, P.hadamard,
                     P.signs, P.k_scale, P.v_scale, P.v_format, P.block_bytes, P.ks_off);
  return hipGetLastError();
}

}  // namespace nvfp4kv
