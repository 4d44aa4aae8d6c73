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
#include "nvfp4kv_rowq.hpp"

namespace nvfp4kv {

namespace {

using namespace rowq;

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
