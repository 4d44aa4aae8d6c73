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

struct PageRegs {
  u4 k[4];   // K codes, tile i: token 16i + (lane%16), dims 32*(lane/16) .. +31
  u4 v[4];   // V codes, load j: token quad 2*(j/2)*4 + (j%2)*4 + lane/16 ... see v_code_word_off
  u4 s;      // 16 bytes of the page's 1 KB of scales (K then V)
};

__device__ inline void load_page(PageRegs& r, const u4* __restrict__ blk, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) r.k[i] = __builtin_nontemporal_load(blk + lane + 64 * i);
#pragma unroll
  for (int i = 0; i < 4; ++i) r.v[i] = __builtin_nontemporal_load(blk + 256 + lane + 64 * i);
  r.s = __builtin_nontemporal_load(blk + 512 + lane);
}

__device__ inline h2 bits_h2(uint32_t b) { return __builtin_bit_cast(h2, b); }

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

__global__ __launch_bounds__(64) void decode_attn_splitk_kernel(
    const uint8_t* __restrict__ pool, int64_t num_pages, int hkv, int layer, int n_q_heads,
    int group, const void* __restrict__ q, int q_dtype, const int32_t* __restrict__ q_positions,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, int rotary_dim,
    int hadamard, const int32_t* __restrict__ page_table, int pt_stride,
    const int32_t* __restrict__ seq_lens, float c_log2, float* __restrict__ ws_acc,
    float2* __restrict__ ws_ml, int pages_per_split, int n_splits) {
  const int split = (int)blockIdx.x, kvh = (int)blockIdx.y, seq = (int)blockIdx.z;
  const int lane = (int)threadIdx.x;
  const int g4 = lane >> 4;     // lane group
  const int c16 = lane & 15;    // column: query head for S/P/O, operand row for K/V
  const int T = seq_lens[seq];
  const int n_pages_seq = (T + kPageSize - 1) / kPageSize;
  const int p0 = split * pages_per_split;
  if (p0 >= n_pages_seq) return;
  const int p1 = min(p0 + pages_per_split, n_pages_seq);

  __shared__ __attribute__((aligned(16))) _Float16 qhat[16 * kHeadDim];
  __shared__ __attribute__((aligned(16))) u4 sc_lds[2][64];

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

  // ---- main loop over the item's pages
  const u4* layer_blocks = reinterpret_cast<const u4*>(
      pool + (size_t)layer * (size_t)num_pages * (size_t)hkv * (size_t)kBlockBytes);
  const int32_t* pt = page_table + (size_t)seq * pt_stride;
  const size_t blk_stride = (size_t)hkv * (kBlockBytes / 16);  // in u4 units
  PageRegs cur, nxt;
  load_page(cur, layer_blocks + (size_t)pt[p0] * blk_stride + (size_t)kvh * (kBlockBytes / 16), lane);

  f4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  for (int p = p0; p < p1; ++p) {
    if (p + 1 < p1)
      load_page(nxt, layer_blocks + (size_t)pt[p + 1] * blk_stride + (size_t)kvh * (kBlockBytes / 16), lane);
    const int buf = (p - p0) & 1;
    sc_lds[buf][lane] = cur.s;
    __syncthreads();
    const uint8_t* scb = reinterpret_cast<const uint8_t*>(&sc_lds[buf][0]);
    const int nvalid = T - p * kPageSize;  // tokens of this page that exist, >= 1

    // ---- QK^T: S[i] holds tokens 16i + 4*g4 + r for query head c16
    f4 S[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * i + c16;
      const uint32_t ku = *reinterpret_cast<const uint16_t*>(scb + t * 8 + 2 * g4);
      const uint32_t s0 = (ku & 0xFFu) << 7, s1 = (ku >> 8) << 7;  // f16 bits of scale * 2^-8
      const h2 sc0 = bits_h2(s0 | (s0 << 16)), sc1 = bits_h2(s1 | (s1 << 16));
      S[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w = cur.k[i][c];
        const h2 sc = (c < 2) ? sc0 : sc1;
        h8 a;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const h2 x = fp4x2(w, b) * sc;
          a[2 * b] = x[0];
          a[2 * b + 1] = x[1];
        }
        S[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[c], S[i], 0, 0, 0);
      }
    }

    // ---- online softmax (log2 domain, weights scaled by 2^15)
    float smax = -INFINITY;
    if (nvalid >= kPageSize) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) smax = fmaxf(smax, S[i][r]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * i + 4 * g4 + r < nvalid) smax = fmaxf(smax, S[i][r]);
    }
    smax = max4lanes(smax);
    const float m_new = fmaxf(m_run, smax * c_log2);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run)) {
      const float alpha = exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= alpha;
      m_run = m_new;
    }
    const float off = 15.0f - m_run;
    float P[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float e = exp2f(fmaf(S[i][r], c_log2, off));
        if (nvalid < kPageSize && 16 * i + 4 * g4 + r >= nvalid) e = 0.0f;
        P[i][r] = e;
        l_run += e;
      }

    // ---- PV over two chunks of 32 tokens
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {
      h8 bhi, blo;
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const float pa = P[2 * ch + (s2 >> 1)][(2 * s2) & 3];
        const float pb = P[2 * ch + (s2 >> 1)][(2 * s2 + 1) & 3];
        const float ha = __uint_as_float(__float_as_uint(pa) & 0xFFFFE000u);
        const float hb = __uint_as_float(__float_as_uint(pb) & 0xFFFFE000u);
        const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(ha, hb));
        const h2 lo = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(pa - ha, pb - hb));
        bhi[2 * s2] = hi[0];
        bhi[2 * s2 + 1] = hi[1];
        blo[2 * s2] = lo[0];
        blo[2 * s2 + 1] = lo[1];
      }
      // V words of the 8 tokens of this lane group; token of k-slot s:
      // s < 4: 32ch + 4*g4 + s, s >= 4: 32ch + 16 + 4*g4 + (s-4)
      const u4 va = cur.v[2 * ch], vb = cur.v[2 * ch + 1];
      const uint32_t w[8] = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
      uint32_t sb[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int t = 32 * ch + (s >= 4 ? 16 : 0) + 4 * g4 + (s & 3);
        uint32_t b = scb[512 + t * 8 + (c16 >> 1)];
        if (t >= nvalid) b = 0;  // stale slot: zero weight and zero value
        sb[s] = b;
      }
      uint32_t A[4], B[4];
      h2 sv[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const uint32_t w0 = w[2 * pr], w1 = w[2 * pr + 1];
        A[pr] = (w0 & 0x0F0F0F0Fu) | ((w1 << 4) & 0xF0F0F0F0u);          // even dims
        B[pr] = ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u);          // odd dims
        sv[pr] = bits_h2((sb[2 * pr] << 7) | (sb[2 * pr + 1] << 23));
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        h8 ae, ao;
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          const h2 e = fp4x2(A[pr], b) * sv[pr];
          const h2 o = fp4x2(B[pr], b) * sv[pr];
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
    }
    cur = nxt;
  }

  // ---- partial results of this item
  const float l_tot = sum4lanes(l_run);
  const size_t item = ((size_t)seq * hkv + kvh) * n_splits + split;
  if (c16 < group) {
    // lane holds dims 32*g4 + 8i + j in acc[j][i]
    float* dst = ws_acc + (item * group + c16) * kHeadDim + 32 * g4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      reinterpret_cast<float4*>(dst + 8 * i)[0] = make_float4(acc[0][i], acc[1][i], acc[2][i], acc[3][i]);
      reinterpret_cast<float4*>(dst + 8 * i)[1] = make_float4(acc[4][i], acc[5][i], acc[6][i], acc[7][i]);
    }
    if (g4 == 0) ws_ml[item * group + c16] = make_float2(m_run, l_tot);
  }
}

// Combine the split partials of one (sequence, query head): 128 threads, one
// output dim each.
__global__ __launch_bounds__(128) void decode_reduce_kernel(
    const float* __restrict__ ws_acc, const float2* __restrict__ ws_ml,
    const int32_t* __restrict__ seq_lens, int hkv, int group, int n_splits, int pages_per_split,
    float* __restrict__ out) {
  const int hq_idx = (int)blockIdx.x;     // query head
  const int seq = (int)blockIdx.y;
  const int d = (int)threadIdx.x;
  const int kvh = hq_idx / group, h = hq_idx % group;
  const int T = seq_lens[seq];
  const int n_pages_seq = (T + kPageSize - 1) / kPageSize;
  const int n_valid = (n_pages_seq + pages_per_split - 1) / pages_per_split;
  const size_t item0 = ((size_t)seq * hkv + kvh) * n_splits;
  float M = -INFINITY;
  for (int s = 0; s < n_valid; ++s) M = fmaxf(M, ws_ml[(item0 + s) * group + h].x);
  float L = 0.0f, o = 0.0f;
  for (int s = 0; s < n_valid; ++s) {
    const float2 ml = ws_ml[(item0 + s) * group + h];
    const float w = exp2f(ml.x - M);
    L += w * ml.y;
    o += w * ws_acc[((item0 + s) * group + h) * kHeadDim + d];
  }
  out[((size_t)seq * hkv * group + hq_idx) * kHeadDim + d] = o / L;
}

}  // namespace

hipError_t launch_decode(const LaunchPool& P, int layer, int n_seq, int n_q_heads, const void* q,
                         int q_dtype, const int32_t* q_positions, const float* rope_cos,
                         const float* rope_sin, const int32_t* page_table, int page_table_stride,
                         const int32_t* seq_lens, float sm_scale, float* out, void* workspace,
                         const DecodePlan& plan, hipStream_t stream) {
  float* ws_acc = reinterpret_cast<float*>(workspace);
  size_t acc_bytes = (ws_acc_bytes(n_seq, P.hkv, plan) + 255) & ~(size_t)255;
  float2* ws_ml = reinterpret_cast<float2*>(reinterpret_cast<uint8_t*>(workspace) + acc_bytes);
  const float c_log2 = sm_scale * 1.4426950408889634f;
  hipLaunchKernelGGL(decode_attn_splitk_kernel, dim3(plan.n_splits, P.hkv, n_seq), dim3(64), 0,
                     stream, P.base, P.num_pages, P.hkv, layer, n_q_heads, plan.group, q, q_dtype,
                     q_positions, rope_cos, rope_sin, P.rotary_dim, P.hadamard, page_table,
                     page_table_stride, seq_lens, c_log2, ws_acc, ws_ml, plan.pages_per_split,
                     plan.n_splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_reduce_kernel, dim3(n_q_heads, n_seq), dim3(128), 0, stream, ws_acc,
                     ws_ml, seq_lens, P.hkv, plan.group, plan.n_splits, plan.pages_per_split, out);
  return hipGetLastError();
}

}  // namespace nvfp4kv
