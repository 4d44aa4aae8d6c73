// Split-K decode attention over the paged NVFP4 KV cache, gfx950.
//
// Method: release post of the gzenz/ninfer fork (prismix.dev), section "NVFP4
// KV cache (from scratch)", bullets 1-2: Q and K are rotated by the Hadamard
// transform and quantized to NVFP4 (E2M1 values, E4M3 scales per 16), QK^T
// runs on the quantized operands, V is stored in NVFP4 and dequantized for
// the PV product.  The post's own QK instruction (a block-scaled FP4 MMA with
// E4M3 scales) has no gfx950 counterpart: the CDNA4 block-scaled MFMA takes
// power-of-two (E8M0) scales per 32 elements.  Here both products dequantize
// in registers to fp16, which holds every E2M1 x E4M3 value exactly, and run
// on v_mfma_f32_16x16x32_f16.
//
// One wavefront (one workgroup) handles a work item (sequence, kv head, range
// of pages).  Per 64-token page it loads 9216 contiguous bytes with nine
// 16-byte loads per lane (the code tiling of the pool makes each load land
// directly in the lane's matrix operand), keeps the next page's loads in
// flight while it computes the current one, and
//   QK  : 4 MFMAs per 16 tokens; A = K-hat (16 tokens x 32 dims per lane
//         group), B = Q-hat (query heads of the group on N, zero-padded to 16)
//   soft: running max per head in log2 units, scores scaled by
//         sm_scale*log2(e), weights 2^(s - m + 15) so that fp16 keeps them
//         normal; reductions across the four lane groups with permlane swaps
//   PV  : O^T[d][h] += V-hat^T[d][t] P^T[t][h]; A = V-hat (16 dims x 32
//         tokens), B = P split into fp16 hi + lo parts (2 MFMAs) so the
//         weights keep ~22 bits.
// Partial (m, l, acc) per item go to the workspace; decode_reduce combines
// them per (sequence, query head).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "nvfp4kv_codec.hpp"
#include "nvfp4kv_internal.hpp"

namespace nvfp4kv {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ inline h2 bits_h2(uint32_t b) { return __builtin_bit_cast(h2, b); }

// Buffer resource over one 9216-byte pool block (raw buffer, gfx9 format
// word); loads past the block's end read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint8_t* blk) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(blk), 0, kBlockBytes, 0x00020000);
}
// 16 bytes at block byte offset voff + soff (voff per lane, soff uniform).
__device__ __forceinline__ u4 ld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}

__device__ inline h2 fp4x2(uint32_t w, int byte_sel) {
  // two E2M1 values of byte `byte_sel` (low nibble first) times 2^8, exact
  switch (byte_sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3);
  }
}

__device__ inline float max4lanes(float v) {
  // max over lanes l, l^16, l^32, l^48
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}

__device__ inline float sum4lanes(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = __int_as_float(a[0]) + __int_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}

// One 32-token half of a page: QK^T for tiles 2hh, 2hh+1, the online
// softmax over those 32 tokens, and PV for them.  `k0`/`k1` hold the two K
// tiles (token 16i + lane%16, dims 32*g4 .. +31), `va`/`vb` the two V token
// quads of this lane group, `sk` this lane's K scale pair of token c16 in the
// staged page (tile stride 128 bytes), `sv` its V scale byte of token 4*g4.
// MASKED halves may hold tokens at or past the sequence end: those get zero
// weight and a zero V scale, chosen by selects so that stale bytes, which may
// decode to NaN, never reach the sums.
template <bool MASKED>
__device__ __forceinline__ void half_step(u4& k0, u4& k1, u4& va, u4& vb, __amdgpu_buffer_rsrc_t nrs,
                                          int voff, const uint8_t* __restrict__ sk,
                                          const uint8_t* __restrict__ sv, int hh, int nvalid,
                                          int g4, const h8 (&qb)[4], float c_log2, f4 (&acc)[8],
                                          float& m_run, float& l_run) {
  // ---- QK^T: S[i] holds tokens 32hh + 16i + 4*g4 + r for query head c16
  f4 S[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t ku = *reinterpret_cast<const uint16_t*>(sk + 128 * (2 * hh + i));
    // f16 bits of (s0 * 2^-8, s1 * 2^-8): an E4M3 byte shifted left by 7 is
    // the f16 encoding of its value times 2^-8 (both subnormal and normal)
    const uint32_t both = (__builtin_amdgcn_perm(0u, ku, 0x0c010c00u)) << 7;
    const h2 sc = bits_h2(both);
    const h2 sc0 = __builtin_shufflevector(sc, sc, 0, 0), sc1 = __builtin_shufflevector(sc, sc, 1, 1);
    const u4& kc = i ? k1 : k0;
    S[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t w = kc[c];
      const h2 scl = (c < 2) ? sc0 : sc1;
      h8 a;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const h2 x = fp4x2(w, b) * scl;
        a[2 * b] = x[0];
        a[2 * b + 1] = x[1];
      }
      S[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[c], S[i], 0, 0, 0);
    }
  }
  // this half's K registers are free: request the next page's.  The loads
  // are unconditional (past a piece's end `nrs` is an empty resource) so that
  // the wait counters stay exact across the loop: a conditional load makes
  // the compiler drain every outstanding load at the join.
  k0 = ld16(nrs, voff, 1024 * (2 * hh));
  k1 = ld16(nrs, voff, 1024 * (2 * hh + 1));

  // ---- online softmax (log2 domain, weights scaled by 2^15)
  float smax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (MASKED) {
        if (32 * hh + 16 * i + 4 * g4 + r < nvalid) smax = fmaxf(smax, S[i][r]);
      } else {
        smax = fmaxf(smax, S[i][r]);
      }
    }
  smax = max4lanes(smax);
  const float m_new = fmaxf(m_run, smax * c_log2);
  if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    m_run = m_new;
  }
  const float off = 15.0f - m_run;
  float P[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float e = __builtin_amdgcn_exp2f(fmaf(S[i][r], c_log2, off));
      if (MASKED && 32 * hh + 16 * i + 4 * g4 + r >= nvalid) e = 0.0f;
      P[i][r] = e;
      l_run += e;
    }

  // ---- PV: O^T[d][h] += V-hat^T[d][t] P^T[t][h] over these 32 tokens; the
  // weights go in as fp16 hi + lo parts (two MFMAs) to keep ~22 bits
  h8 bhi, blo;
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    const float pa = P[s2 >> 1][(2 * s2) & 3];
    const float pb = P[s2 >> 1][(2 * s2 + 1) & 3];
    const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(pa, pb));
    const float ra = pa - (float)hi[0];     // exact remainders
    const float rb = pb - (float)hi[1];
    const h2 lo = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(ra, rb));
    bhi[2 * s2] = hi[0];
    bhi[2 * s2 + 1] = hi[1];
    blo[2 * s2] = lo[0];
    blo[2 * s2 + 1] = lo[1];
  }
  // V words of the 8 tokens of this lane group; token of k-slot s:
  // s < 4: 32hh + 4*g4 + s, s >= 4: 32hh + 16 + 4*g4 + (s-4)
  const uint32_t w[8] = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
  uint32_t A[4], B[4];
  h2 svp[4];
#pragma unroll
  for (int pr = 0; pr < 4; ++pr) {
    const uint32_t w0 = w[2 * pr], w1 = w[2 * pr + 1];
    A[pr] = (w0 & 0x0F0F0F0Fu) | ((w1 << 4) & 0xF0F0F0F0u);   // even dims
    B[pr] = ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u);   // odd dims
    const int s0 = 2 * pr, s1 = 2 * pr + 1;
    const int t0 = 32 * hh + (s0 >= 4 ? 16 : 0) + (s0 & 3);   // token offset from 4*g4
    const int t1 = 32 * hh + (s1 >= 4 ? 16 : 0) + (s1 & 3);
    uint32_t b0 = sv[8 * t0], b1 = sv[8 * t1];
    if (MASKED) {
      if (t0 + 4 * g4 >= nvalid) b0 = 0;   // stale slot: zero value
      if (t1 + 4 * g4 >= nvalid) b1 = 0;
    }
    svp[pr] = bits_h2((b0 | (b1 << 16)) << 7);
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    h8 ae, ao;
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      const h2 e = fp4x2(A[pr], b) * svp[pr];
      const h2 o = fp4x2(B[pr], b) * svp[pr];
      ae[2 * pr] = e[0];
      ae[2 * pr + 1] = e[1];
      ao[2 * pr] = o[0];
      ao[2 * pr + 1] = o[1];
    }
    acc[2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, bhi, acc[2 * b], 0, 0, 0);
    acc[2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, blo, acc[2 * b], 0, 0, 0);
    acc[2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao, bhi, acc[2 * b + 1], 0, 0, 0);
    acc[2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao, blo, acc[2 * b + 1], 0, 0, 0);
  }
  // and the V registers: request the next page's
  va = ld16(nrs, voff, kVCodeOff + 1024 * (2 * hh));
  vb = ld16(nrs, voff, kVCodeOff + 1024 * (2 * hh + 1));
}

// Pages of sequence `s`.
__device__ inline int64_t seq_pages(const int32_t* __restrict__ seq_lens, int s) {
  return (seq_lens[s] + kPageSize - 1) / kPageSize;
}

// The wave whose range [w*TP/W, (w+1)*TP/W) holds flattened page index x.
__device__ inline int64_t wave_of(int64_t x, int64_t TP, int64_t W) { return ((x + 1) * W - 1) / TP; }

// One piece of work: pages [p0, p1) of (seq, kvh).  Writes (m, l, acc) for
// the group's query heads to partial slot `slot`.
__device__ __forceinline__ void decode_piece(
    const uint8_t* __restrict__ pool, int64_t num_pages, int hkv, int layer, int n_q_heads,
    int group, const void* __restrict__ q, int q_dtype, const int32_t* __restrict__ q_positions,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, int rotary_dim,
    int hadamard, const int32_t* __restrict__ page_table, int pt_stride, int T, float c_log2,
    float* __restrict__ ws_acc, float2* __restrict__ ws_ml, int seq, int kvh, int p0, int p1,
    size_t slot, _Float16* qhat, u4 (*sc_lds)[64]) {
  const int lane = (int)threadIdx.x;
  const int g4 = lane >> 4;     // lane group
  const int c16 = lane & 15;    // column: query head for S/P/O, operand row for K/V

  // ---- query prologue: RoPE, Hadamard, NVFP4 round trip, fp16 Q-hat in LDS
  for (int pass = 0; pass < (group + 3) / 4; ++pass) {
    const int h = pass * 4 + g4;
    const int hh = h < group ? h : group - 1;
    const size_t off = ((size_t)seq * n_q_heads + (size_t)kvh * group + hh) * kHeadDim + 8 * c16;
    float x[8];
    if (q_dtype == 1) {
      const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(q) + off);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(u[i] << 16);
        x[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q) + off);
      const float4 a = p[0], b = p[1];
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    const float* crow = nullptr;
    const float* srow = nullptr;
    if (rotary_dim > 0) {
      const int pos = q_positions[seq];
      crow = rope_cos + (size_t)pos * (rotary_dim / 2);
      srow = rope_sin + (size_t)pos * (rotary_dim / 2);
    }
    uint32_t codes, scode;
    quant_row16(x, c16, rotary_dim, crow, srow, hadamard != 0, codes, scode);
    const float s = e4m3_value(scode);
    h8 qv;
#pragma unroll
    for (int k = 0; k < 8; ++k) qv[k] = (_Float16)(e2m1_value((codes >> (4 * k)) & 15u) * s);
    if (h < group) *reinterpret_cast<h8*>(&qhat[h * kHeadDim + 8 * c16]) = qv;
  }
  __syncthreads();
  h8 qb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    h8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    qb[c] = (c16 < group) ? *reinterpret_cast<const h8*>(&qhat[c16 * kHeadDim + 32 * g4 + 8 * c]) : z;
  }

  // ---- main loop over the piece's pages
  const uint8_t* layer_base =
      pool + (size_t)layer * (size_t)num_pages * (size_t)hkv * (size_t)kBlockBytes;
  const int32_t* pt = page_table + (size_t)seq * pt_stride;
  const size_t blk_stride = (size_t)hkv * kBlockBytes;
  const int voff = 16 * lane;
  // One page in registers at a time.  Each half-page's K codes are requested
  // for the next page as soon as QK^T has consumed them, its V codes as soon
  // as PV has, and the scales right after the current ones went to LDS, so
  // every load overlaps the rest of the current page.
  __amdgpu_buffer_rsrc_t rs = block_rsrc(layer_base + (size_t)pt[p0] * blk_stride + (size_t)kvh * kBlockBytes);
  // Issued in the order the loop issues them (scales, then K and V of each
  // half), so the wait counts at the loop head are the same on entry and on
  // the back edge.
  u4 kc[4], vc[4], sc;
  sc = ld16(rs, voff, kKScaleOff);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    kc[2 * hh] = ld16(rs, voff, 1024 * (2 * hh));
    kc[2 * hh + 1] = ld16(rs, voff, 1024 * (2 * hh + 1));
    __builtin_amdgcn_sched_barrier(0);
    vc[2 * hh] = ld16(rs, voff, kVCodeOff + 1024 * (2 * hh));
    vc[2 * hh + 1] = ld16(rs, voff, kVCodeOff + 1024 * (2 * hh + 1));
    __builtin_amdgcn_sched_barrier(0);
  }

  f4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  // lane-invariant LDS byte offsets of this lane's scales inside a staged page
  const int sk_off = 8 * c16 + 2 * g4;            // K scales of token c16 (+16i), blocks 2g4, 2g4+1
  const int sv_off = 512 + 32 * g4 + (c16 >> 1);  // V scales of token 4*g4 (+...), block c16/2
  for (int p = p0; p < p1; ++p) {
    // the next page; past the piece's end an empty resource (loads return
    // zeros without memory traffic) keeps the load sequence unchanged
    const bool more = p + 1 < p1;
    const __amdgpu_buffer_rsrc_t nrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(layer_base + (size_t)pt[more ? p + 1 : p] * blk_stride + (size_t)kvh * kBlockBytes),
        0, more ? kBlockBytes : 0, 0x00020000);
    const int buf = (p - p0) & 1;
    sc_lds[buf][lane] = sc;
    __syncthreads();
    sc = ld16(nrs, voff, kKScaleOff);
    const uint8_t* scb = reinterpret_cast<const uint8_t*>(&sc_lds[buf][0]);
    const int nvalid = T - p * kPageSize;  // tokens of this page that exist, >= 1
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      // each half's registers are refilled with the next page's data as soon
      // as this half has consumed them (inside half_step)
      if (nvalid >= kPageSize)
        half_step<false>(kc[2 * hh], kc[2 * hh + 1], vc[2 * hh], vc[2 * hh + 1], nrs, voff,
                         scb + sk_off, scb + sv_off, hh, nvalid, g4, qb, c_log2, acc, m_run, l_run);
      else
        half_step<true>(kc[2 * hh], kc[2 * hh + 1], vc[2 * hh], vc[2 * hh + 1], nrs, voff,
                        scb + sk_off, scb + sv_off, hh, nvalid, g4, qb, c_log2, acc, m_run, l_run);
    }
  }

  // ---- partial results of this piece
  const float l_tot = sum4lanes(l_run);
  if (c16 < group) {
    // lane holds dims 32*g4 + 8i + j in acc[j][i]
    float* dst = ws_acc + (slot * group + c16) * kHeadDim + 32 * g4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      reinterpret_cast<float4*>(dst + 8 * i)[0] = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
      reinterpret_cast<float4*>(dst + 8 * i)[1] = make_float4(acc[4][i], acc[5][i], acc[6][i], acc[7][i]);
    }
    if (g4 == 0) ws_ml[slot * group + c16] = make_float2(m_run, l_tot);
  }
  __syncthreads();  // the next piece rewrites qhat
}

// Stream-K decode.  All (sequence, kv head, page) work is laid out flat:
// segment g = seq * hkv + kvh holds that pair's pages, segments in order.
// With TP pages in all and W = gridDim.x wavefronts, wave w takes the range
// [w*TP/W, (w+1)*TP/W), so every wave gets the same number of pages (+-1)
// whatever the sequence lengths.  A range may start or end inside a segment
// and may cover several; the wave writes one partial per segment piece, to
// slot g + w (distinct for every (segment, wave) pair that overlaps).
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_attn_splitk_kernel(
    const uint8_t* __restrict__ pool, int64_t num_pages, int hkv, int layer, int n_seq,
    int n_q_heads, int group, const void* __restrict__ q, int q_dtype,
    const int32_t* __restrict__ q_positions, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, int rotary_dim, int hadamard,
    const int32_t* __restrict__ page_table, int pt_stride, const int32_t* __restrict__ seq_lens,
    float c_log2, float* __restrict__ ws_acc, float2* __restrict__ ws_ml) {
  __shared__ __attribute__((aligned(16))) _Float16 qhat[16 * kHeadDim];
  __shared__ __attribute__((aligned(16))) u4 sc_lds[2][64];

  const int64_t W = gridDim.x, w = blockIdx.x;
  int64_t TP = 0;
  for (int s = 0; s < n_seq; ++s) TP += seq_pages(seq_lens, s);
  TP *= hkv;
  int64_t x = (w * TP) / W;
  const int64_t end = ((w + 1) * TP) / W;
  if (x >= end) return;
  // find the sequence holding x
  int seq = 0;
  int64_t seq_base = 0;  // flat index of the first page of seq's first segment
  int64_t pg = seq_pages(seq_lens, 0);
  while (x >= seq_base + hkv * pg) {
    seq_base += hkv * pg;
    ++seq;
    pg = seq_pages(seq_lens, seq);
  }
  while (x < end) {
    const int kvh = (int)((x - seq_base) / pg);
    const int64_t seg_start = seq_base + kvh * pg;
    const int p0 = (int)(x - seg_start);
    const int64_t seg_end = seg_start + pg;
    const int p1 = (int)((end < seg_end ? end : seg_end) - seg_start);
    const size_t slot = (size_t)seq * hkv + kvh + (size_t)w;
    decode_piece(pool, num_pages, hkv, layer, n_q_heads, group, q, q_dtype, q_positions, rope_cos,
                 rope_sin, rotary_dim, hadamard, page_table, pt_stride, seq_lens[seq], c_log2,
                 ws_acc, ws_ml, seq, kvh, p0, p1, slot, qhat, sc_lds);
    x = seg_start + p1;
    if (kvh == hkv - 1 && x < end) {
      seq_base += hkv * pg;
      ++seq;
      pg = seq_pages(seq_lens, seq);
    }
  }
}

// Combine the partials of one (sequence, query head) for 32 output dims:
// 256 threads = 32 dims x 8 groups that stride over the pieces.  The pieces
// of segment g come from waves w_first .. w_last, found with the same flat
// indexing as the decode kernel; waves with an empty range (more waves than
// pages) wrote nothing and are skipped.
__global__ __launch_bounds__(256) void decode_reduce_kernel(
    const float* __restrict__ ws_acc, const float2* __restrict__ ws_ml,
    const int32_t* __restrict__ seq_lens, int n_seq, int hkv, int group, int64_t W,
    float* __restrict__ out) {
  const int hq_idx = (int)blockIdx.x;     // query head
  const int seq = (int)blockIdx.y;
  const int d0 = 32 * (int)blockIdx.z;    // first output dim of this block
  const int tid = (int)threadIdx.x;
  const int dd = tid & 31, j = tid >> 5;  // dim within the chunk, piece group
  const int kvh = hq_idx / group, h = hq_idx % group;
  int64_t TP = 0, seq_base = 0;
  for (int s = 0; s < n_seq; ++s) {
    const int64_t pg = seq_pages(seq_lens, s);
    if (s == seq) seq_base = TP;
    TP += pg;
  }
  TP *= hkv;
  seq_base *= hkv;
  const int64_t pg = seq_pages(seq_lens, seq);
  const int64_t S = seq_base + kvh * pg, E = S + pg;
  const int64_t w0 = wave_of(S, TP, W), w1 = wave_of(E - 1, TP, W);
  const size_t g = (size_t)seq * hkv + kvh;

  constexpr int kChunk = 1024;             // pieces whose weights are staged at once
  __shared__ float red_m[8];
  __shared__ float red_o[8][32];
  __shared__ float red_l[8];
  __shared__ float wts[kChunk];
  // ---- running max over all pieces
  float M = -INFINITY;
  for (int64_t w = w0 + tid; w <= w1; w += 256) {
    if ((w * TP) / W == ((w + 1) * TP) / W) continue;
    M = fmaxf(M, ws_ml[(g + w) * group + h].x);
  }
  for (int o = 16; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 32));
  if ((tid & 31) == 0) red_m[tid >> 5] = M;
  __syncthreads();
  M = red_m[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) M = fmaxf(M, red_m[i]);

  // ---- weighted sums, a chunk of pieces at a time: weights 2^(m - M) go to
  // LDS once, then 8 groups stride over the pieces with 16 independent loads
  // in flight per thread
  float L = 0.0f, acc = 0.0f;
  for (int64_t c0 = w0; c0 <= w1; c0 += kChunk) {
    const int n = (int)((w1 - c0 + 1) < kChunk ? (w1 - c0 + 1) : kChunk);
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const int64_t w = c0 + i;
      float wt = 0.0f;
      if ((w * TP) / W != ((w + 1) * TP) / W) {
        const float2 ml = ws_ml[(g + w) * group + h];
        wt = exp2f(ml.x - M);
        L += wt * ml.y;
      }
      wts[i] = wt;
    }
    __syncthreads();
    for (int i = j; i < n; i += 128) {
      float a[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int iu = i + 8 * u < n ? i + 8 * u : i;
        a[u] = ws_acc[((g + c0 + iu) * group + h) * kHeadDim + d0 + dd];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (i + 8 * u < n) acc += wts[i + 8 * u] * a[u];
    }
  }
  // L was summed per thread over its pieces; combine across the block
  for (int o = 16; o > 0; o >>= 1) L += __shfl_xor(L, o, 32);
  red_o[j][dd] = acc;
  if (dd == 0) red_l[j] = L;
  __syncthreads();
  if (j == 0) {
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o += red_o[i][dd];
      l += red_l[i];
    }
    out[((size_t)seq * hkv * group + hq_idx) * kHeadDim + d0 + dd] = o / l;
  }
}

}  // namespace

hipError_t launch_decode_splits(const LaunchPool& P, int layer, int n_seq, int n_q_heads,
                                const void* q, int q_dtype, const int32_t* q_positions,
                                const float* rope_cos, const float* rope_sin,
                                const int32_t* page_table, int page_table_stride,
                                const int32_t* seq_lens, float sm_scale, void* workspace,
                                const DecodePlan& plan, hipStream_t stream) {
  float* ws_acc = reinterpret_cast<float*>(workspace);
  const size_t acc_bytes = (ws_acc_bytes(n_seq, P.hkv, plan) + 255) & ~(size_t)255;
  float2* ws_ml = reinterpret_cast<float2*>(reinterpret_cast<uint8_t*>(workspace) + acc_bytes);
  const float c_log2 = sm_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(decode_attn_splitk_kernel, dim3(plan.n_waves), dim3(64), 0, stream, P.base,
                     P.num_pages, P.hkv, layer, n_seq, n_q_heads, plan.group, q, q_dtype,
                     q_positions, rope_cos, rope_sin, P.rotary_dim, P.hadamard, page_table,
                     page_table_stride, seq_lens, c_log2, ws_acc, ws_ml);
  return hipGetLastError();
}

hipError_t launch_decode_reduce(int hkv, int n_seq, int n_q_heads, const int32_t* seq_lens,
                                float* out, const void* workspace, const DecodePlan& plan,
                                hipStream_t stream) {
  const float* ws_acc = reinterpret_cast<const float*>(workspace);
  const size_t acc_bytes = (ws_acc_bytes(n_seq, hkv, plan) + 255) & ~(size_t)255;
  const float2* ws_ml =
      reinterpret_cast<const float2*>(reinterpret_cast<const uint8_t*>(workspace) + acc_bytes);
  hipLaunchKernelGGL(decode_reduce_kernel, dim3(n_q_heads, n_seq, kHeadDim / 32), dim3(256), 0, stream, ws_acc,
                     ws_ml, seq_lens, n_seq, hkv, plan.group, (int64_t)plan.n_waves, out);
  return hipGetLastError();
}

int decode_waves_per_cu() {
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, decode_attn_splitk_kernel, 64, 0) != hipSuccess)
    return 0;
  return blocks;
}

}  // namespace nvfp4kv
