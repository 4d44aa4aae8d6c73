// Row quantizer of the fused kernels for gfx950: one 128-element row on 16
// lanes (8 elements each), RoPE, the Hadamard transform's cross-lane stages
// through DPP, the E4M3 block scale and the E2M1 codes, bit for bit what
// quant_row16 (nvfp4kv_codec.hpp) computes.  Used by the append kernel for
// K rows and by the decode kernels for the query rows, which go through the
// same NVFP4 round trip: release post of the gzenz/ninfer fork (prismix.dev),
// section "NVFP4 KV cache (from scratch)", bullets 1 and 2.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4kv_codec.hpp"

namespace nvfp4kv {
namespace rowq {

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

// One cross-lane stage of the transform, exact in every case (signed zeros
// included): the lower lane of a pair keeps a + b, the upper one a - b (its
// partner's value minus its own), as one fused multiply-add by +-1, which
// rounds exactly as the addition or subtraction does.
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

// Cross-lane stages of the transform (strides 8, 16, 32 and 64: lane bits
// 0-3 of the row), each a DPP instruction per element, one for bits 0, 1
// and 3 and two for bit 2.  For bits 0, 1 and 3 every lane adds its
// partner's value times +1 (lower lane) or -1 (upper lane) to its own in one
// fused multiply-add, which rounds exactly as the sum or difference does, so
// the upper lane holds the negated difference.  A lane's sign so far then
// depends only on the lane bits of the stages before, which both lanes of a
// later pair share, so every later stage computes the signed sum or
// difference of the true values; the sign (-1)^(r0 + r1 + r3) is folded into
// the closing multiply by 1/sqrt(128).  Signed zeros: the held value of a
// zero is +0 whatever its sign so far (a cancellation rounds to +0), and so
// is the true value as long as no -0 enters the transform (-0 only comes
// from -0 operands); the closing fma(h, +-c, +0) then gives +0 for every
// zero, as the plain transform does.  Rows with a -0 input take the stages
// above instead.  For bit 2 the lower lanes (banks 0
// and 2 of the row) take partner + own and the upper ones partner - own,
// each under a bank mask.  Each block starts with 5 wait states: a DPP
// source written by a VALU (or EXEC written by SALU) just before needs them.
#define NVFP4KV_DPP8(OP, CTRL)                                                       \
  "s_nop 4\n\t" OP " %0, %0, %8 " CTRL "\n\t" OP " %1, %1, %8 " CTRL "\n\t" OP  \
  " %2, %2, %8 " CTRL "\n\t" OP " %3, %3, %8 " CTRL "\n\t" OP " %4, %4, %8 " CTRL \
  "\n\t" OP " %5, %5, %8 " CTRL "\n\t" OP " %6, %6, %8 " CTRL "\n\t" OP         \
  " %7, %7, %8 " CTRL
#define NVFP4KV_X8(x) "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7])

__device__ __forceinline__ void fwht_cross_lanes(float (&x)[8], int r) {
  const float s0 = (r & 1) ? -1.0f : 1.0f, s1 = (r & 2) ? -1.0f : 1.0f, s3 = (r & 8) ? -1.0f : 1.0f;
  asm(NVFP4KV_DPP8("v_fmac_f32_dpp", "quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1")
      : NVFP4KV_X8(x) : "v"(s0));
  asm(NVFP4KV_DPP8("v_fmac_f32_dpp", "quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1")
      : NVFP4KV_X8(x) : "v"(s1));
  float y[8];
#define NVFP4KV_PM4(I, J)                                                      \
  "v_add_f32_dpp %" I ", %" J ", %" J " row_shl:4 row_mask:0xf bank_mask:0x5\n\t" \
  "v_sub_f32_dpp %" I ", %" J ", %" J " row_shr:4 row_mask:0xf bank_mask:0xa\n\t"
  asm("s_nop 4\n\t" NVFP4KV_PM4("0", "8") NVFP4KV_PM4("1", "9") NVFP4KV_PM4("2", "10") NVFP4KV_PM4("3", "11")
          NVFP4KV_PM4("4", "12") NVFP4KV_PM4("5", "13") NVFP4KV_PM4("6", "14") NVFP4KV_PM4("7", "15")
      : "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]), "=&v"(y[4]), "=&v"(y[5]), "=&v"(y[6]), "=&v"(y[7])
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]));
#undef NVFP4KV_PM4
  asm(NVFP4KV_DPP8("v_fmac_f32_dpp", "row_ror:8 row_mask:0xf bank_mask:0xf bound_ctrl:1")
      : NVFP4KV_X8(y) : "v"(s3));
  const float sg = ((r ^ (r >> 1) ^ (r >> 3)) & 1) ? -1.0f : 1.0f;
  const float c = sg * __uint_as_float(0x3DB504F3u);   // +-(float nearest 1/sqrt(128))
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] = __builtin_fmaf(y[k], c, 0.0f);
}
#undef NVFP4KV_DPP8
#undef NVFP4KV_X8

// E2M1 codes of a lane's 8 values for block scale s, packed (value k in bits
// 4k..4k+3).  Magnitudes by a three-level search over the same exact
// thresholds as e2m1_code: 1.75s (>=) splits codes 0-3 from 4-7, then 0.75s
// or 3.5s (>=), then 0.25s, 1.25s, 2.5s or 5s (>).  The thresholds increase
// and each test is monotone in |y|, so the result is the count of thresholds
// passed, as in e2m1_code; with s = 0 every threshold is +infinity and every
// magnitude code 0.  Selects only, no branches; the seven thresholds are
// made once and kept in registers.  Sign bits are gathered with byte
// permutes: the top byte of each even value into one word, of each odd value
// into another, then shifted and masked into bit 3 of each nibble.
__device__ __forceinline__ uint32_t e2m1_codes8(const float (&x)[8], float s) {
  if (s == 0.0f) s = __builtin_inff();
  float T[7] = {0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.0f * s};
#pragma unroll
  for (int i = 0; i < 7; ++i) asm volatile("" : "+v"(T[i]));
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float a = fabsf(x[k]);
    const bool b2 = a >= T[3];
    const float t1 = b2 ? T[5] : T[1];
    const float lo = b2 ? T[4] : T[0], hi = b2 ? T[6] : T[2];
    const bool b1 = a >= t1;
    const bool b0 = a > (b1 ? hi : lo);
    uint32_t m = (uint32_t)b2;
    m = m + m + (uint32_t)b1;
    m = m + m + (uint32_t)b0;
    w |= m << (4 * k);
  }
  const uint32_t u0 = __float_as_uint(x[0]), u1 = __float_as_uint(x[1]), u2 = __float_as_uint(x[2]),
                 u3 = __float_as_uint(x[3]), u4 = __float_as_uint(x[4]), u5 = __float_as_uint(x[5]),
                 u6 = __float_as_uint(x[6]), u7 = __float_as_uint(x[7]);
  // byte j of `ev`: the top byte of value 2j; of `od`: of value 2j + 1
  const uint32_t ev = __builtin_amdgcn_perm(u2, u0, 0x0C0C0703u) | (__builtin_amdgcn_perm(u6, u4, 0x0C0C0703u) << 16);
  const uint32_t od = __builtin_amdgcn_perm(u3, u1, 0x0C0C0703u) | (__builtin_amdgcn_perm(u7, u5, 0x0C0C0703u) << 16);
  return w | ((ev >> 4) & 0x08080808u) | (od & 0x80808080u);
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
                                             const RopeLane& rl, bool hadamard, uint32_t neg, bool neg_any,
                                             uint32_t& codes, uint32_t& scode) {
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
    if (neg_any) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if ((neg >> k) & 1u) x[k] = -x[k];
    }
    // a -0 among the wavefront's inputs (its bit pattern is the least int)
    int lo = min(min(__float_as_int(x[0]), __float_as_int(x[1])), __float_as_int(x[2]));
    lo = min(min(lo, __float_as_int(x[3])), __float_as_int(x[4]));
    lo = min(min(lo, __float_as_int(x[5])), __float_as_int(x[6]));
    lo = min(lo, __float_as_int(x[7]));
    const bool neg_zero = __builtin_amdgcn_ballot_w64(lo == (int)0x80000000) != 0;
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
    if (__builtin_expect(neg_zero, 0)) {
      fwht_stage<1>(x, r);
      fwht_stage<2>(x, r);
      fwht_stage<4>(x, r);
      fwht_stage<8>(x, r);
      const float inv_sqrt128 = __uint_as_float(0x3DB504F3u);
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = x[k] * inv_sqrt128;
    } else {
      fwht_cross_lanes(x, r);
    }
  }
  float am = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) am = fmaxf(am, fabsf(x[k]));
  am = fmaxf(am, xor_lane<1>(am));
  codes = e2m1_codes8(x, e4m3_scale_fast(am, scode));
}

}  // namespace rowq
}  // namespace nvfp4kv
