// Device-side NVFP4 codec for gfx950: RoPE, 128-point Hadamard rotation and
// E4M3/E2M1 quantization of one 128-element row held by 16 lanes of a
// wavefront (8 consecutive elements per lane).
//
// Method: release post of the gzenz/ninfer fork (prismix.dev), section
// "NVFP4 KV cache (from scratch)", bullets 1-2 (E2M1 values with E4M3 block
// scales; Hadamard rotation of K and Q before quantization) and section
// "YaRN context extension" (rotary part of the head, theta, linear scaling).
//
// The floating-point steps that decide codes are written so that every
// operation is one IEEE binary32 operation in a fixed order, with contraction
// into fused multiply-adds switched off: RoPE products and sums rounded one by
// one, the fast Walsh-Hadamard transform in ascending strides 1..64 with
// (a, b) -> (a + b, a - b), then one multiply by the float nearest 1/sqrt(128).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4kv {

constexpr int kHeadDim = 128;
constexpr int kPageSize = 64;
constexpr int kBlockBytes = 9216;   // one (layer, page, kv head) block
constexpr int kKCodeOff = 0;
constexpr int kVCodeOff = 4096;
constexpr int kKScaleOff = 8192;
constexpr int kVScaleOff = 8704;
// Blocks of a pool that keeps V in fp16 (v_format 1): K codes as above, the
// fp16 V tiles at kVCodeOff, then the K scales.
constexpr int kBlockBytesF16V = 20992;
constexpr int kKScaleOffF16V = 20480;

// Byte offset, inside a block, of the 4-byte word holding code bytes
// 4w .. 4w+3 of token t (w = 0..15).
__host__ __device__ inline uint32_t k_code_word_off(uint32_t t, uint32_t w) {
  return kKCodeOff + (t / 16) * 1024 + (w / 4) * 256 + (t % 16) * 16 + (w % 4) * 4;
}
__host__ __device__ inline uint32_t v_code_word_off(uint32_t t, uint32_t w) {
  return kVCodeOff + (t / 4) * 256 + w * 16 + (t % 4) * 4;
}

// Byte offset, inside an fp16-V block, of V element d of token t.  Unit
// u = t/32 of the page holds 8 tiles of 1 KB, tile j the dims d with
// d % 8 == j; in a tile, the 16 bytes at 16 * (g4*16 + d/8) hold the eight
// tokens 4*g4 + r and 16 + 4*g4 + r (r = 0..3) of the unit, in that order:
// the A operand of one lane of the PV matrix instruction.
__host__ __device__ inline uint32_t v16_off(uint32_t t, uint32_t d) {
  return kVCodeOff + (t / 32) * 8192 + (d % 8) * 1024 + (((t % 16) / 4) * 16 + d / 8) * 16 +
         ((t % 4) + 4 * ((t % 32) / 16)) * 2;
}

// binary16 bits of x, nearest with ties to even (the conversion instruction
// rounds so in the default mode; overflow gives infinity).
__device__ inline uint32_t f16_bits(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// E4M3 code of the scale for a block with largest magnitude `amax`: the E4M3
// value nearest amax/6, ties to the even code, 448 (0x7E) on overflow.
// fl32(amax/6) rounds to the same E4M3 value as the exact quotient: the
// E4M3 decision points have at most 5 significant bits, so the quotient can
// only sit on one when amax = 6 * point exactly, in which case the division
// is exact too.
__host__ __device__ inline uint32_t e4m3_scale_code(float amax) {
  const float x = amax / 6.0f;               // correctly rounded division
  if (!(x < 448.0f)) return 0x7Eu;           // also catches x == 448
  if (x < 0.015625f) {                       // below 2^-6: steps of 2^-9
    const float m = rintf(x * 512.0f);       // exact scaling, round half even
    return (uint32_t)m;                      // 0..8; 8 is 2^-6 (code 0x08)
  }
  uint32_t bits = __float_as_uint(x);
  // keep 3 mantissa bits, round to nearest even; a carry moves the exponent
  bits = bits + 0x7FFFFu + ((bits >> 20) & 1u);
  bits &= 0xFFF00000u;
  const uint32_t e = (bits >> 23) & 0xFFu;   // biased fp32 exponent, >= 121
  const uint32_t m = (bits >> 20) & 7u;
  return ((e - 120u) << 3) | m;              // E4M3 bias 7 = 127 - 120
}

// The same block scale (code and value, equal to e4m3_scale_code and
// e4m3_value of it for every non-negative binary32 amax, +infinity
// included) in a few operations and no branch.  amax/6: q0 = amax * fl(1/6)
// corrected once with the exact remainder amax - 6 q0 (two fused
// multiply-adds); this is the correctly rounded quotient except where it is
// subnormal, far below the smallest scale.  Rounding to the E4M3 grid (3
// mantissa bits, spacing 2^-9 below 2^-6) by adding and subtracting
// M = 1.5 * 2^(e + 20), e the quotient's exponent clamped to [-6, 8]: the sum
// lands in M's binade, whose spacing is the grid's, so the addition rounds to
// the grid (nearest, ties to even) and the subtraction is exact.  Values
// from 464 up round to 480 or more and saturate to 448.  The code follows
// from the value's bits (normal) or value * 2^9 (subnormal).
__host__ __device__ inline float e4m3_scale_fast(float amax, uint32_t& code) {
#pragma clang fp contract(off)
  const float c6 = 0x1.555556p-3f;           // the float nearest 1/6
  const float q0 = amax * c6;
  const float x = fmaf(fmaf(-q0, 6.0f, amax), c6, q0);
  uint32_t eb = __builtin_bit_cast(uint32_t, x) >> 23;
  eb = eb < 121u ? 121u : eb > 135u ? 135u : eb;
  const float m = __builtin_bit_cast(float, ((eb + 20u) << 23) | 0x400000u);
  float s = (x + m) - m;
  s = fminf(s, 448.0f);
  code = s >= 0.015625f ? (__builtin_bit_cast(uint32_t, s) >> 20) - 960u : (uint32_t)(s * 512.0f);
  return s;
}

// E4M3 code -> float (exact).  Codes are never NaN here.
__host__ __device__ inline float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;      // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 magnitude code of |y| for block scale s, nearest with ties to the even
// code: the products t*s below are exact in binary32 (t has at most 3
// significant bits, s at most 4), so each comparison is exact.
__host__ __device__ inline uint32_t e2m1_code(float y, float s) {
  const float a = fabsf(y);
  uint32_t c = (uint32_t)(a > 0.25f * s) + (uint32_t)(a >= 0.75f * s) +
               (uint32_t)(a > 1.25f * s) + (uint32_t)(a >= 1.75f * s) +
               (uint32_t)(a > 2.5f * s) + (uint32_t)(a >= 3.5f * s) + (uint32_t)(a > 5.0f * s);
  if (s == 0.0f) c = 0;
  return c | (signbit(y) ? 8u : 0u);
}

__host__ __device__ inline float e2m1_value(uint32_t nib) {
  const uint32_t m = nib & 7u;
  // 0, .5, 1, 1.5, 2, 3, 4, 6
  const float mag = (m < 2) ? 0.5f * (float)m : (float)((2u + (m & 1u)) << ((m >> 1) - 1u)) * 0.5f;
  return (nib & 8u) ? -mag : mag;
}

// Elements elem_off .. +7 of a bf16 (dtype 1) or f32 (dtype 0) array as floats,
// with one 16-byte load (bf16) or two (f32).
__device__ inline void load8(const void* src, int dtype, size_t elem_off, float (&x)[8]) {
  if (dtype == 1) {  // bf16
    const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(src) + elem_off);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(u[i] << 16);
      x[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + elem_off);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// RoPE coefficients of a lane's 8 elements for quant_row16_v: lane r of a
// row covers elements e = 8r .. 8r+7; in the first half of the rotary part
// (e < R/2) it needs cos/sin of pair e, in the second half those of pair
// e - R/2, beyond the rotary part nothing (zeros are returned, and not used).
// GR (general rotary widths): any even R, element by element; otherwise R is
// a multiple of 16 and a lane's 8 coefficients are consecutive.
template <bool GR = false>
__device__ inline void rope_coeffs(int r, int rotary_dim, const float* cos_row, const float* sin_row,
                                   float (&cv)[8], float (&sv)[8]) {
  const int half = rotary_dim / 2;
  if constexpr (GR) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int e = 8 * r + k;
      const int idx = e < half ? e : e - half;
      cv[k] = e < rotary_dim ? cos_row[idx] : 0.0f;
      sv[k] = e < rotary_dim ? sin_row[idx] : 0.0f;
    }
  } else {
    const int hl = half / 8;                  // lanes per half
    const bool in_rot = r < 2 * hl;
    const int base = in_rot ? (r < hl ? 8 * r : 8 * r - half) : 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      cv[k] = in_rot ? cos_row[base + k] : 0.0f;
      sv[k] = in_rot ? sin_row[base + k] : 0.0f;
    }
  }
}

// Rotate-half RoPE on a row held 8 elements per lane by a 16-lane row, for a
// half-width R/2 = 8*hl + D that is not a multiple of 8.  Element e = 8r + k
// pairs with e + R/2 (first half) or e - R/2 (second half): element
// (k + D) % 8 of lane r + hl (+1 when k + D >= 8), or element (k - D) % 8 of
// lane r - hl (-1 when k < D).  D is a template argument, so the registers
// exchanged are fixed; both partners are fetched for every element (every
// lane takes part in every shuffle) and the element's own half picks one.
// Each product and each sum is rounded on its own, as in quant_row16_v.
template <int D>
__device__ __forceinline__ void rope_rows_general(float (&x)[8], int r, int half, const float (&cv)[8],
                                                  const float (&sv)[8]) {
#pragma clang fp contract(off)
  const int base = (int)__lane_id() & ~15;
  const int hl = half >> 3;
  float fw[8], bw[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int lf = min(r + hl + ((k + D) >> 3), 15);       // lanes past the row are not used
    const int lb = max(r - hl - (k < D ? 1 : 0), 0);
    fw[k] = __shfl(x[(k + D) & 7], base + lf, 64);
    bw[k] = __shfl(x[(k + 8 - D) & 7], base + lb, 64);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int e = 8 * r + k;
    if (e < half) {
      const float ac = x[k] * cv[k];
      const float bs = fw[k] * sv[k];
      x[k] = ac - bs;
    } else if (e < 2 * half) {
      const float bc = x[k] * cv[k];
      const float as = bw[k] * sv[k];
      x[k] = bc + as;
    }
  }
}

// rope_rows_general for D = half % 8 in 1..7.
__device__ __forceinline__ void rope_rows_any(float (&x)[8], int r, int half, const float (&cv)[8],
                                              const float (&sv)[8]) {
  switch (half & 7) {
    case 1: rope_rows_general<1>(x, r, half, cv, sv); break;
    case 2: rope_rows_general<2>(x, r, half, cv, sv); break;
    case 3: rope_rows_general<3>(x, r, half, cv, sv); break;
    case 4: rope_rows_general<4>(x, r, half, cv, sv); break;
    case 5: rope_rows_general<5>(x, r, half, cv, sv); break;
    case 6: rope_rows_general<6>(x, r, half, cv, sv); break;
    default: rope_rows_general<7>(x, r, half, cv, sv); break;
  }
}

// Quantize one 128-element row held by the 16 lanes of a lane group.  GR:
// any even rotary width (the general rotation); otherwise the width is a
// multiple of 16 (0 included), the only case the code then holds.  `x`
// holds elements 8r .. 8r+7 of the row, r = lane % 16; `cv`/`sv` the lane's
// RoPE coefficients from rope_coeffs (unused when rotary_dim is 0).  On
// return `x` holds the rotated (RoPE'd, Hadamard'd) floats, `codes` the
// lane's 8 E2M1 codes (element 8r+k in bits 4k..4k+3) and `scode` the E4M3
// code of the lane's block (elements 16(r/2) .. 16(r/2)+15).  With the
// rotation, the elements whose bit is set in `neg` (bit k: element 8r+k; the
// randomized rotation's mask, else 0) are negated before it.  All 64 lanes of
// the wavefront must call it together (it uses cross-lane shuffles).
template <bool GR = false>
__device__ inline void quant_row16_v(float (&x)[8], int r, int rotary_dim, const float (&cv)[8],
                                     const float (&sv)[8], bool hadamard, uint32_t neg,
                                     uint32_t& codes, uint32_t& scode) {
#pragma clang fp contract(off)
  const int lane = (int)__lane_id();
  // RoPE, rotate-half pairs (i, i + R/2) on the first R dims.
  if (GR && rotary_dim > 0 && (rotary_dim & 15) != 0) {
    rope_rows_any(x, r, rotary_dim / 2, cv, sv);
  } else if (rotary_dim > 0) {
    const int half = rotary_dim / 2;
    const int hl = half / 8;
    const bool first = r < hl;
    const bool second = (r >= hl) && (r < 2 * hl);
    const int src = first ? r + hl : (second ? r - hl : r);
    const int src_lane = (lane & ~15) + src;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float other = __shfl(x[k], src_lane, 64);
      if (first) {
        const float ac = x[k] * cv[k];
        const float bs = other * sv[k];
        x[k] = ac - bs;
      } else if (second) {
        const float bc = x[k] * cv[k];
        const float as = other * sv[k];
        x[k] = bc + as;
      }
    }
  }
  if (hadamard) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if ((neg >> k) & 1u) x[k] = -x[k];
    // strides 1, 2, 4 inside the lane
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
    // strides 8, 16, 32, 64 across lanes r ^ 1, r ^ 2, r ^ 4, r ^ 8
#pragma unroll
    for (int bit = 1; bit < 16; bit <<= 1) {
      const bool upper = (r & bit) != 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p = __shfl_xor(x[k], bit, 64);
        x[k] = upper ? (p - x[k]) : (x[k] + p);
      }
    }
    const float inv_sqrt128 = __uint_as_float(0x3DB504F3u);  // nearest float to 2^-3.5
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = x[k] * inv_sqrt128;
  }
  float am = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(x[k]));
  am = fmaxf(am, __shfl_xor(am, 1, 64));
  scode = e4m3_scale_code(am);
  const float s = e4m3_value(scode);
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) w |= e2m1_code(x[k], s) << (4 * k);
  codes = w;
}

// quant_row16_v with the RoPE coefficients read from the table rows.
template <bool GR = false>
__device__ inline void quant_row16(float (&x)[8], int r, int rotary_dim, const float* cos_row,
                                   const float* sin_row, bool hadamard, uint32_t neg, uint32_t& codes,
                                   uint32_t& scode) {
  float cv[8], sv[8];
  if (rotary_dim > 0) {
    rope_coeffs<GR>(r, rotary_dim, cos_row, sin_row, cv, sv);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) cv[k] = sv[k] = 0.0f;
  }
  quant_row16_v<GR>(x, r, rotary_dim, cv, sv, hadamard, neg, codes, scode);
}

}  // namespace nvfp4kv
