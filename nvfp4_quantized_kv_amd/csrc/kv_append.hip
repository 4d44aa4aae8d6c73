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

// A lane's 8 inputs of a row as raw words: bf16 (DT 1) takes 4 words, f32
// (DT 0) 8.
template <int DT>
struct RawRow {
  uint32_t w[DT == 1 ? 4 : 8];
};

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

// One workgroup (8 wavefronts) per range of tokens, in passes of 16 tokens:
// wavefronts 0-3 take the K rows of a pass (4 tokens each, one row of 16
// lanes per token), 4-7 its V rows, so every wavefront's rows are all K or
// all V and only K rows run RoPE and the rotation.  A wavefront goes through
// the kv heads of its 4 tokens before the next pass: RoPE coefficients are
// read once per pass, and a row's input address differs from the one before
// by a constant.  The inputs of the next row are loaded before the current
// row is quantized, so their latency overlaps its arithmetic.
//
// Ranges follow the pool's line groups.  A line group is 16 slots of a page
// from a multiple of 16; per (page, kv head) block it owns whole 128-byte
// lines (1024 bytes of K codes, 1024 of V codes, 128 of each scale) that no
// other slot touches.  Workgroup w takes tokens [a_w, a_{w+1}), a_w the first
// token from 64w on that starts a line group (its slot a multiple of 16, or
// not the slot after the previous token's), which lies within 16 tokens of
// 64w; its passes start at a_w, so the 16 tokens of a group are quantized
// in one pass and their lines filled at once.  No line is then written by
// two workgroups (unless the slots jump inside a group) nor in two pieces
// far apart in time; either way a line goes back to HBM in pieces, and
// 64-token ranges that ignored the groups cost a seventh more write traffic
// than the bytes.  The slots and positions of the 80 tokens from 64w are
// read once, in the same round trip as the range's bounds, and each pass
// takes its tokens' from the lanes that hold them.
template <int DT, bool GR>
__global__ __launch_bounds__(512) void kv_quant_append_kernel(
    uint8_t* __restrict__ pool, int64_t num_pages, int hkv, int layer, int n_tok,
    const void* __restrict__ k, const void* __restrict__ v,
    const int64_t* __restrict__ slots, const int32_t* __restrict__ positions,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, int rotary_dim,
    int hadamard, SignMask signs, float k_inv, float v_inv, int v_format, int block_bytes, int ks_off) {
  const int lane = (int)__lane_id();
  const int r = lane & 15;
  // the wavefront's index, made wave-uniform for the compiler: every choice
  // derived from it (K or V rows, the transform, the fp16 V store) is then a
  // scalar branch rather than masked lanes
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int which = wv >> 2;                       // 0 = K, 1 = V
  const bool vf16 = which && v_format;             // V rows kept in fp16
  const int rot = which ? 0 : rotary_dim;
  const bool had = which ? false : (hadamard != 0);
  const uint32_t neg = which ? 0u : lane_signs(hadamard, signs, r);
  const bool neg_any = !which && hadamard == 2;    // the randomized rotation's negations
  const float inv = which ? v_inv : k_inv;         // 1 / the global scale
  const int lt0 = (wv & 3) * 4 + (lane >> 4);      // the lane's token within a pass

  // the window: tokens 64w + lane (wa) and 64w + 64 + lane (wb, lanes 0-15),
  // with the slot of the token before each
  const int w64 = (int)blockIdx.x * 64;
  const int ia = min(w64 + lane, n_tok - 1), ib = min(w64 + 64 + (lane & 15), n_tok - 1);
  const int64_t sa = slots[ia], sb = slots[ib];
  const int64_t pa = slots[max(ia - 1, 0)], pb = slots[max(ib - 1, 0)];
  const int qa = rot > 0 ? positions[ia] : 0, qb = rot > 0 ? positions[ib] : 0;
  // a line-group start before token i (slot s, previous slot sp)
  auto starts = [&](int i, int64_t s, int64_t sp) { return i <= 0 || i >= n_tok || s % 16 == 0 || s != sp + 1; };
  const uint64_t sm = __builtin_amdgcn_ballot_w64(lane < 16 ? starts(w64 + lane, sa, pa)
                                                  : lane < 32 ? starts(w64 + 64 + (lane & 15), sb, pb) : false);
  const int ra = min(w64 + (int)__builtin_ctzll((sm & 0xFFFFull) | 0x10000ull), n_tok);
  const int rb = min(w64 + 64 + (int)__builtin_ctzll(((sm >> 16) & 0xFFFFull) | 0x10000ull), n_tok);
  const int n_pass = (rb - ra + 15) / 16;          // at most 5: a range holds at most 79 tokens
  // the lane's token in pass p (lanes past the range take its last token's
  // rows: they still take part in the cross-lane steps, and store nothing),
  // with its slot and position from the window
  auto token = [&](int p, bool& valid, int64_t& slot, int& pos) {
    const int t = ra + 16 * p + lt0;
    valid = t < rb;
    const int tc = valid ? t : rb - 1;
    const int j = tc - w64;                        // 0 .. 78
    const int src = (j & 63) << 2;
    const int lo = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)sa);
    const int hi = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(sa >> 32));
    const int lo2 = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)sb);
    const int hi2 = __builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(sb >> 32));
    slot = j < 64 ? (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo)
                  : (int64_t)(((uint64_t)(uint32_t)hi2 << 32) | (uint32_t)lo2);
    pos = 0;
    if (rot > 0) {
      const int p1 = __builtin_amdgcn_ds_bpermute(src, qa), p2 = __builtin_amdgcn_ds_bpermute(src, qb);
      pos = j < 64 ? p1 : p2;
    }
    return tc;
  };

  const size_t row_elems = (size_t)hkv * kHeadDim;
  constexpr int kEs = DT == 1 ? 2 : 4;             // input element bytes
  const char* src = reinterpret_cast<const char*>(which ? v : k);
  auto load_row = [&](const char* ptr, RawRow<DT>& rw) {
    if (DT == 1) {
      const uint4 q = *reinterpret_cast<const uint4*>(ptr);
      rw.w[0] = q.x; rw.w[1] = q.y; rw.w[2] = q.z; rw.w[3] = q.w;
    } else {
      const uint4 a = reinterpret_cast<const uint4*>(ptr)[0], b = reinterpret_cast<const uint4*>(ptr)[1];
      rw.w[0] = a.x; rw.w[1] = a.y; rw.w[2] = a.z; rw.w[3] = a.w;
      rw.w[4] = b.x; rw.w[5] = b.y; rw.w[6] = b.z; rw.w[7] = b.w;
    }
  };
  // the lane's 8 inputs of kv head g of token t
  auto row_ptr = [&](int t, int g) { return src + ((size_t)t * row_elems + (size_t)g * kHeadDim + 8 * r) * kEs; };

#pragma unroll 1
  for (int g0 = 0; g0 < hkv; g0 += 4) {
    const int G = min(4, hkv - g0);
    bool valid;
    int64_t slot;
    int pos;
    const char* rp = row_ptr(token(0, valid, slot, pos), g0);
    RawRow<DT> rw;
    load_row(rp, rw);
#pragma unroll 1
    for (int p = 0; p < n_pass; ++p) {
      const bool active = valid;
      RopeLane rl;
      if (rot > 0)
        rope_lane<GR>(r, rotary_dim, rope_cos + (size_t)pos * (rotary_dim / 2),
                      rope_sin + (size_t)pos * (rotary_dim / 2), rl);
      // the next pass's token
      bool valid_n;
      int64_t slot_n;
      int pos_n;
      const char* rp_n = row_ptr(token(min(p + 1, n_pass - 1), valid_n, slot_n, pos_n), g0);
      const uint32_t t = (uint32_t)(slot % kPageSize);
      const uint32_t woff = which ? v_code_word_off(t, (uint32_t)r) : k_code_word_off(t, (uint32_t)r);
      const uint32_t soff = (which ? kVScaleOff : ks_off) + 8 * t + r / 2;
      uint8_t* blk0 = pool + (((size_t)layer * (size_t)num_pages + (size_t)(slot / kPageSize)) * (size_t)hkv + g0) *
                                 (size_t)block_bytes;
#pragma unroll 1
      for (int gl = 0; gl < G; ++gl) {
        __builtin_amdgcn_sched_barrier(0);
        RawRow<DT> rw_n;
        load_row(gl + 1 < G ? rp + (size_t)(gl + 1) * kHeadDim * kEs : rp_n, rw_n);
        __builtin_amdgcn_sched_barrier(0);
        float x[8];
        raw_to_float<DT>(rw, x);
        if (inv != 1.0f) {   // (x * 1 is x: the common case skips it)
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] *= inv;
        }
        uint8_t* blk = blk0 + (size_t)gl * (size_t)block_bytes;
        if (vf16) {
          // V kept in fp16: element 8r + e rounded to nearest even, into its tile
          // (element 8r + e sits at the lane's offset plus 1024 e)
          if (active) {
            uint16_t* vb = reinterpret_cast<uint16_t*>(blk + v16_off(t, (uint32_t)(8 * r)));
#pragma unroll
            for (int e = 0; e < 8; ++e) vb[512 * e] = (uint16_t)f16_bits(x[e]);
          }
        } else {
          uint32_t codes, scode;
          append_row16<GR>(x, r, rot > 0, rot, rl, had, neg, neg_any, codes, scode);
          if (active) {
            *reinterpret_cast<uint32_t*>(blk + woff) = codes;
            if ((r & 1) == 0) blk[soff] = (uint8_t)scode;
          }
        }
        rw = rw_n;
      }
      valid = valid_n;
      slot = slot_n;
      pos = pos_n;
      rp = rp_n;
    }
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
