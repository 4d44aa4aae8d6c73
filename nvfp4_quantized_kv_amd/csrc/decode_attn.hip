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
// The decode kernel splits the pages of all (sequence, kv head) pairs evenly
// over its wavefronts (one workgroup each, all resident).  Each wavefront
// quantizes the queries of the pairs it covers into MFMA operands in LDS
// (and, when given, the step's new token into the cache), then streams its
// range page by page: per 64-token page it
// loads 9216 contiguous bytes with nine 16-byte loads per lane (the code
// tiling of the pool makes each load land directly in the lane's matrix
// operand), two pages ahead of use, and
//   QK  : 4 MFMAs per 16 tokens; A = K-hat (16 tokens x 32 dims per lane
//         group), B = Q-hat (query heads of the group on N)
//   soft: per-head reference in log2 units, scores scaled by
//         sm_scale*log2(e), weights 2^(s - m + 8) kept below 2^15 so that
//         fp16 keeps them normal; reductions across the four lane groups
//         with permlane swaps, only when the reference has to move
//   PV  : O^T[d][h] += V-hat^T[d][t] P^T[t][h]; A = V-hat (16 dims x 32
//         tokens), B = the weights split into fp16 high and low parts, so
//         they keep ~22 bits (for groups of up to 8 heads both parts share
//         one MFMA: columns 0-7 carry the high parts, 8-15 the low parts).
// Groups of up to 8 heads take the softmax a page at a time: the QK^T of a
// page's two units land in the two halves of each 16-lane row (the query
// operand's other half zeroed), so one pass of exponentials covers 64 tokens.
// Partial (m, l, acc) per (pair, wavefront) go to the workspace;
// decode_reduce combines them per (sequence, query head).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "nvfp4kv_codec.hpp"
#include "nvfp4kv_internal.hpp"
#include "nvfp4kv_rowq.hpp"

// This file is compiled twice: as is, for rotary widths that are multiples
// of 16 (the kernels the workloads run), and from decode_attn_gr.hip with
// NVFP4KV_DECODE_GENERAL_ROPE 1, whose kernels also take every other even
// width.  Keeping the general rotation out of the first build keeps it out
// of those kernels' register allocation.
#ifndef NVFP4KV_DECODE_GENERAL_ROPE
#define NVFP4KV_DECODE_GENERAL_ROPE 0
#endif

namespace nvfp4kv {

constexpr bool kGR = NVFP4KV_DECODE_GENERAL_ROPE != 0;

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ inline h2 bits_h2(uint32_t b) { return __builtin_bit_cast(h2, b); }

// a - (float)h for the f16 h in the low (HI false) or high half of a pair,
// in one mixed-precision fused multiply-add: the f16 operand converts
// exactly, so this rounds once, as the conversion and subtraction do
// (the compiler emits those two instructions for the plain expression)
template <bool HI>
__device__ __forceinline__ float sub_f16(float a, h2 h) {
  float d;
  if (HI)
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(a));
  else
    asm("v_fma_mix_f32 %0, -%1, 1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(a));
  return d;
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

// The online softmax works in log2 units: a score s (already multiplied by
// sm_scale * log2(e)) gets the weight 2^(s - m + kOff), where m is a per-head
// reference that is raised only when some score passes m + kMargin.  Weights
// therefore stay below 2^(kOff + kMargin) = 2^15, inside fp16's normal range,
// and most 32-token units skip the cross-lane maximum and the rescale.
constexpr float kOff = 8.0f;
constexpr float kMargin = 7.0f;

// QK^T of one 32-token unit (K tiles i = 0, 1 of the unit): S[t][i] holds
// tokens 16i + 4*g4 + r of the unit for query column 16t + c16 (t < NT
// column tiles, each dequantized K operand feeding NT MFMAs).  `k0`/`k1`
// hold the lane's 32 codes of token c16 (+16) for dims 32*g4 .. +31; `sk`
// points at the lane's K scale pair (blocks 2*g4, 2*g4+1) of the unit's
// first token row in the staged page (tile stride 128 bytes).
template <int NT, bool ACCUM = false>
__device__ __forceinline__ void qk_unit(const u4& k0, const u4& k1, const uint8_t* __restrict__ sk,
                                        const h8 (&qb)[NT][4], f4 (&S)[NT][2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t ku = *reinterpret_cast<const uint16_t*>(sk + 128 * i);
    // f16 bits of (s0 * 2^-8, s1 * 2^-8): an E4M3 byte shifted left by 7 is
    // the f16 encoding of its value times 2^-8 (both subnormal and normal)
    const h2 sc = bits_h2(__builtin_amdgcn_perm(0u, ku, 0x0c010c00u) << 7);
    const h2 sc0 = __builtin_shufflevector(sc, sc, 0, 0), sc1 = __builtin_shufflevector(sc, sc, 1, 1);
    const u4& kc = i ? k1 : k0;
    if (!ACCUM)
#pragma unroll
      for (int t = 0; t < NT; ++t) S[t][i] = f4{0.f, 0.f, 0.f, 0.f};
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
#pragma unroll
      for (int t = 0; t < NT; ++t) S[t][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[t][c], S[t][i], 0, 0, 0);
    }
  }
}

// PV of one 32-token unit: O^T[d][h] += V-hat^T[d][t] P^T[t][h].  `va`/`vb`
// hold the V codes of tokens 4*g4 + r and 16 + 4*g4 + r of the unit (dims
// 8*c16 .. +7); `sv` points at the V scale byte of the unit's token 4*g4,
// block c16/2, in the staged page.  PACKED: `p0` carries the fp16 high part
// of the weights in columns 0-7 and the low part in columns 8-15, one MFMA
// per tile; otherwise `p0`/`p1` are the high/low parts, two MFMAs per tile.
// With NT column tiles every dequantized V operand feeds all of them.
template <bool PACKED, int NT>
__device__ __forceinline__ void pv_unit(const u4& va, const u4& vb, const uint8_t* __restrict__ sv,
                                        const h8 (&p0)[NT], const h8 (&p1)[NT], f4 (&acc)[NT][8]) {
  // V words of the 8 tokens of this lane group; token of k-slot s:
  // s < 4: 4*g4 + s, s >= 4: 16 + 4*g4 + (s-4)
  const uint32_t w[8] = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
  uint32_t A[4], B[4];
  h2 svp[4];
#pragma unroll
  for (int pr = 0; pr < 4; ++pr) {
    const uint32_t w0 = w[2 * pr], w1 = w[2 * pr + 1];
    A[pr] = (w0 & 0x0F0F0F0Fu) | ((w1 << 4) & 0xF0F0F0F0u);   // even dims
    B[pr] = ((w0 >> 4) & 0x0F0F0F0Fu) | (w1 & 0xF0F0F0F0u);   // odd dims
    const int t0 = (pr >= 2 ? 16 : 0) + 2 * (pr & 1);          // token offset from 4*g4
    const uint32_t b0 = sv[8 * t0], b1 = sv[8 * (t0 + 1)];
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
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[t][2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, p0[t], acc[t][2 * b], 0, 0, 0);
      acc[t][2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao, p0[t], acc[t][2 * b + 1], 0, 0, 0);
      if (!PACKED) {
        acc[t][2 * b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ae, p1[t], acc[t][2 * b], 0, 0, 0);
        acc[t][2 * b + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao, p1[t], acc[t][2 * b + 1], 0, 0, 0);
      }
    }
  }
}

// PV of one 32-token unit with V kept in fp16 (v_format 1): `vh` holds the
// lane's A operands of the unit's 8 dim tiles (tile j: dims 8*c16 + j of the
// tokens of k-slots 0-7, as the pool's fp16 tiling stores them), so the
// operands go to the matrix instructions as loaded.  Weights as in pv_unit.
template <bool PACKED, int NT>
__device__ __forceinline__ void pv_unit_f16(const u4 (&vh)[8], const h8 (&p0)[NT], const h8 (&p1)[NT],
                                            f4 (&acc)[NT][8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const h8 a = __builtin_bit_cast(h8, vh[j]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p0[t], acc[t][j], 0, 0, 0);
      if (!PACKED) acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, p1[t], acc[t][j], 0, 0, 0);
    }
  }
}

// fp16 V of a page's tokens nv .. 63 set to zero in the lane's operands (both
// units): a slot past a sequence's end may hold any bytes, Inf or NaN among
// them, and a zero weight does not cancel those in the matrix product.
__device__ __forceinline__ void mask_v16(u4 (&vh)[16], int nv, int g4) {
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // k-slots 2w and 2w+1: tokens 32u + 4*g4 + s (s < 4) or 32u + 12 + 4*g4 + s (s >= 4)
      const int s0 = 2 * w, s1 = 2 * w + 1;
      const int t0 = 32 * u + 4 * g4 + s0 + (s0 >= 4 ? 12 : 0);
      const int t1 = 32 * u + 4 * g4 + s1 + (s1 >= 4 ? 12 : 0);
      const uint32_t m = (t0 < nv ? 0x0000FFFFu : 0u) | (t1 < nv ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int j = 0; j < 8; ++j) vh[8 * u + j][w] &= m;
    }
}

// Pages of sequence `s`.
__device__ inline int64_t seq_pages(const int32_t* __restrict__ seq_lens, int s) {
  return (seq_lens[s] + kPageSize - 1) / kPageSize;
}

// The wave whose range [w*TU/W, (w+1)*TU/W) holds work unit x.
__device__ inline int64_t wave_of(int64_t x, int64_t TU, int64_t W) { return ((x + 1) * W - 1) / TU; }

// Work units of the stream-K split: every segment counts its pages plus
// kSegExtra units of no work after its last page.  The wavefront whose
// range holds a segment's end (it quantizes the current token there and
// switches segments) thereby gets that many fewer pages; measured, those
// wavefronts otherwise finish 10-25 us after the median one.
constexpr int kSegExtra = 5;

// Flattened page index (pages of all segments in order) of the first page at
// or after work unit u; u = total units gives the total page count.
__device__ inline int64_t page_of_unit(int64_t u, const int32_t* __restrict__ seq_lens, int n_seq,
                                       int hkv) {
  int64_t P = 0, U = 0;
  for (int s = 0; s < n_seq; ++s) {
    const int64_t pg = seq_pages(seq_lens, s);
    const int64_t span = (int64_t)hkv * (pg + kSegExtra);
    if (u < U + span) {
      const int64_t k = (u - U) / (pg + kSegExtra);
      const int64_t off = (u - U) - k * (pg + kSegExtra);
      return P + k * pg + min(off, pg);
    }
    U += span;
    P += (int64_t)hkv * pg;
  }
  return P;
}

// The sequences' page counts and the flat unit and page offsets of their
// first segments, held across the wavefront: lane l of chunk c stands for
// sequence 64c + l.  The lengths are read 8 per round trip and the offsets
// are prefix sums by lane shuffles, so the lookups below are ballots and
// register reads, where a walk over the sequences took one dependent load
// per step (with 64 sequences, 40-110 us of a wavefront's start).  From
// kWalkSeqs + 1 up to kScanSeqs sequences; otherwise the walks.
// (vector types, not arrays: an array indexed in a loop before unrolling is
// moved to LDS, one LDS round trip per access)
constexpr int kScanChunks = 4;
constexpr int kScanSeqs = 64 * kScanChunks;
// Up to this many sequences the walks are cheaper (measured: three
// sequences, 2.0 us to a wavefront's range against 2.5 us for the scan).
constexpr int kWalkSeqs = 4;
typedef int scan_i4 __attribute__((ext_vector_type(4)));
typedef int64_t scan_l4 __attribute__((ext_vector_type(4)));
struct SeqScan {
  scan_i4 pg;   // per chunk: pages of the lane's sequence (0 past n_seq)
  scan_l4 u0;   // flat unit index of its first segment
  scan_l4 p0;   // flat page index of its first page
  int64_t TU, TP;   // units and pages of all segments
};

__device__ __forceinline__ int64_t readlane64(int64_t x, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), l);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void seq_scan(const int32_t* __restrict__ seq_lens, int n_seq, int hkv, SeqScan& sc) {
  const int lane = (int)__lane_id();
  // the lengths through the scalar cache, 8 independent loads per wait,
  // set into the lanes: every wavefront reads the same words at its start,
  // and as one vector load per wavefront that hot line took 3-13 us
  scan_i4 len;
#pragma unroll
  for (int c = 0; c < kScanChunks; ++c) {
    len[c] = 0;
    if (64 * c < n_seq) {
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int base = 64 * c + 8 * g;
        if (base < n_seq) {
          int v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = seq_lens[min(base + i, n_seq - 1)];
#pragma unroll
          for (int i = 0; i < 8; ++i) len[c] = lane == 8 * g + i ? v[i] : len[c];
        }
      }
    }
  }
  int64_t uc = 0, pc = 0;
#pragma unroll
  for (int c = 0; c < kScanChunks; ++c) {
    const int sq = 64 * c + lane;
    const int pg = sq < n_seq ? (len[c] + kPageSize - 1) / kPageSize : 0;
    const int64_t u = sq < n_seq ? (int64_t)hkv * (pg + kSegExtra) : 0;
    const int64_t p = (int64_t)hkv * pg;
    int64_t ui = u, pi = p;
    // (only the steps the chunk's sequences need; lanes past them keep
    // partial sums, which are never read)
    const int nc = min(n_seq - 64 * c, 64);
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      if (d >= nc) break;
      const int64_t ut = __shfl_up(ui, d, 64), pt = __shfl_up(pi, d, 64);
      if (lane >= d) {
        ui += ut;
        pi += pt;
      }
    }
    sc.pg[c] = pg;
    sc.u0[c] = uc + ui - u;
    sc.p0[c] = pc + pi - p;
    if (nc > 0) {   // the chunk's totals: its last sequence's inclusive sums
      uc += readlane64(ui, nc - 1);
      pc += readlane64(pi, nc - 1);
    }
  }
  sc.TU = uc;
  sc.TP = pc;
}

// Chunk c (wave-uniform or per lane) of a scanned array.
template <typename V>
__device__ __forceinline__ auto scan_chunk(const V& v, int c) {
  auto r = v[0];
#pragma unroll
  for (int k = 1; k < kScanChunks; ++k) r = c == k ? v[k] : r;
  return r;
}

// Entry `src` (a lane index) of chunk c of a scanned array, c chosen per
// lane: every chunk in use is shuffled and the reading lane picks its own
// (a shuffle of an array chosen per lane would return the chunk the source
// lane chose).
template <typename V>
__device__ __forceinline__ auto scan_shfl(const V& v, int c, int src, int n_seq) {
  auto r = __shfl(v[0], src, 64);
#pragma unroll
  for (int k = 1; k < kScanChunks; ++k)
    if (64 * k < n_seq) {
      const auto t = __shfl(v[k], src, 64);
      r = c == k ? t : r;
    }
  return r;
}

// Sequence s's page count and first unit / page (s wave-uniform, < n_seq).
__device__ __forceinline__ int scan_pages(const SeqScan& sc, int s) {
  return __builtin_amdgcn_readlane(scan_chunk(sc.pg, s >> 6), s & 63);
}

// The last sequence whose offset `off` (its first unit or page) is at or
// before x; sequences with no pages share the offset of the next one, so
// for a page x this is the sequence holding it.
__device__ __forceinline__ int scan_seq_at(const scan_l4& off, int64_t x, int n_seq) {
  const int lane = (int)__lane_id();
  int n = 0;
#pragma unroll
  for (int c = 0; c < kScanChunks; ++c)
    n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(64 * c + lane < n_seq && off[c] <= x));
  return n - 1;
}

// page_of_unit from the scan.
__device__ __forceinline__ int64_t scan_page_of_unit(const SeqScan& sc, int64_t u, int n_seq) {
  if (u >= sc.TU) return sc.TP;
  const int sq = scan_seq_at(sc.u0, u, n_seq);
  const int64_t U = readlane64(scan_chunk(sc.u0, sq >> 6), sq & 63);
  const int64_t P = readlane64(scan_chunk(sc.p0, sq >> 6), sq & 63);
  const int64_t pg = scan_pages(sc, sq);
  const int64_t k = (u - U) / (pg + kSegExtra);
  const int64_t off = (u - U) - k * (pg + kSegExtra);
  return P + k * pg + min(off, pg);
}

// Per lane: the sequence holding flat page x (x < TP), by a binary search
// over the scanned first pages (every lane runs the same shuffle steps).
__device__ __forceinline__ int scan_seq_of_page_lane(const SeqScan& sc, int64_t x, int n_seq) {
  // chunk: the last one whose first sequence starts at or before x
  int c = 0;
#pragma unroll
  for (int k = 1; k < kScanChunks; ++k)
    if (64 * k < n_seq && readlane64(sc.p0[k], 0) <= x) c = k;
  const int nv = min(n_seq - 64 * c, 64);   // valid lanes of the chunk
  // (steps below the largest chunk in use: the others probe past its end)
  const int span = min(n_seq, 64);
  int lo = 0;
#pragma unroll
  for (int step = 32; step >= 1; step >>= 1) {
    if (step >= span) continue;
    const int probe = lo + step;
    const int64_t v = scan_shfl(sc.p0, c, probe & 63, n_seq);
    if (probe < nv && v <= x) lo = probe;
  }
  return 64 * c + lo;
}

// Query columns.  A kernel pass works on `group` columns per kv head: the
// query heads of the kv head (`heads` of them) for `group / heads`
// consecutive query tokens starting at token qtok0 of the n_qtok new tokens
// of each sequence (one token, qtok0 0 and group == heads for a plain
// decode).  Column c is head c % heads of token qtok0 + c / heads; q and out
// are laid out [seq][token][query head][128].
struct QCols {
  int group, heads, n_qtok, qtok0;
};

// Inputs of one segment's query operands: the query rows of the columns (up
// to 4 per pass, one 16-lane group per column) and the lane's RoPE
// coefficients at the segment's one position; with several query tokens
// (MQ) the rows' positions instead, their coefficients being loaded per pass
// when the operands are made (one set per pass would hold 16 more registers
// per pass through the page loads).
// A lane's query inputs as loaded: the 8 elements of each pass as raw
// words (bf16: w[.][0]; f32: both), unpacked only where the operands are
// made, so no instruction waits for these loads before the first page loads
// are issued (the wait counter is in order: a load read early would be
// waited for with everything issued before it).
template <int kPasses, bool MQ>
struct QIn {
  u4 w[kPasses][2];
  u4 rc[2], rs[2];   // RoPE cos / sin of the lane's 8 elements, as loaded
  int pos[MQ ? kPasses : 1];
  int dtype;
};

__device__ __forceinline__ void q_unpack(const u4 (&w)[2], int dtype, float (&x)[8]) {
  if (dtype == 1) {   // bf16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[0][i] << 16);
      x[2 * i + 1] = __uint_as_float(w[0][i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(w[0][i]);
      x[4 + i] = __uint_as_float(w[1][i]);
    }
  }
}

// RoPE coefficients of a lane's 8 query elements (those of rope_coeffs), as
// loaded: lanes past the rotary part read the row's first 8 pairs, which the
// rotation does not use, instead of taking zeros, so nothing selects on (and
// waits for) these loads before the rotation itself.  Rows of R/2 floats,
// R a multiple of 16, start on 32-byte boundaries.
template <bool GR>
__device__ __forceinline__ void rope_coeffs_q(int r, int rotary_dim, const float* __restrict__ cos_row,
                                              const float* __restrict__ sin_row, u4 (&rc)[2], u4 (&rs)[2]) {
  if constexpr (GR) {
    float cv[8], sv[8];
    rope_coeffs<true>(r, rotary_dim, cos_row, sin_row, cv, sv);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      rc[k / 4][k % 4] = __float_as_uint(cv[k]);
      rs[k / 4][k % 4] = __float_as_uint(sv[k]);
    }
  } else {
    const int half = rotary_dim / 2, hl = half / 8;
    const int base = r < hl ? 8 * r : r < 2 * hl ? 8 * r - half : 0;
    rc[0] = *reinterpret_cast<const u4*>(cos_row + base);
    rc[1] = *reinterpret_cast<const u4*>(cos_row + base + 4);
    rs[0] = *reinterpret_cast<const u4*>(sin_row + base);
    rs[1] = *reinterpret_cast<const u4*>(sin_row + base + 4);
  }
}

template <int kPasses, bool MQ>
__device__ __forceinline__ void load_q_inputs(int sg, int hkv, int n_q_heads, const QCols& qc,
                                              const void* __restrict__ q, int q_dtype,
                                              const int32_t* __restrict__ q_positions,
                                              const float* __restrict__ rope_cos,
                                              const float* __restrict__ rope_sin, int rotary_dim,
                                              QIn<kPasses, MQ>& in) {
  const int lane = (int)threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  const int seq = sg / hkv, kvh = sg % hkv;
  in.dtype = q_dtype;
  const bool bf16 = q_dtype == 1;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int col = min(pass * 4 + g4, qc.group - 1);
    const int tok = MQ ? qc.qtok0 + col / qc.heads : 0;
    const int h = MQ ? col % qc.heads : col;
    const size_t e0 =
        (((size_t)seq * (MQ ? qc.n_qtok : 1) + tok) * n_q_heads + (size_t)kvh * qc.heads + h) * kHeadDim +
        8 * c16;
    // the lane's 16 (bf16) or 32 (f32) bytes; bf16 reads its 16 twice
    const uint8_t* p0 = static_cast<const uint8_t*>(q) + e0 * (bf16 ? 2 : 4);
    in.w[pass][0] = *reinterpret_cast<const u4*>(p0);
    in.w[pass][1] = *reinterpret_cast<const u4*>(bf16 ? p0 : p0 + 16);
    if (MQ) in.pos[pass] = rotary_dim > 0 ? q_positions[(size_t)seq * qc.n_qtok + tok] : 0;
  }
  if (!MQ) {
    // loaded on both sides of the rotary test (no join to copy them across,
    // which would wait for them): without RoPE the query rows stand in for
    // the table, read and not used
    const int pos = rotary_dim > 0 ? q_positions[seq] : 0;
    const float* qf = static_cast<const float*>(q);
    rope_coeffs_q<kGR>(c16, rotary_dim, rotary_dim > 0 ? rope_cos + (size_t)pos * (rotary_dim / 2) : qf,
                       rotary_dim > 0 ? rope_sin + (size_t)pos * (rotary_dim / 2) : qf, in.rc, in.rs);
  }
}

// Entries per row of a query-operand slot in LDS: one per lane, then a zero
// entry (read by lanes whose operand columns are to be zero).  For groups
// of up to 8 heads (PACKED) lanes c16 and c16 + 8 take the same operand: one
// entry per (g4, c16 % 8), 32 of them, then the zero entry.
template <bool PACKED>
constexpr int q_entries() { return PACKED ? 33 : 65; }

// Query operands of one segment into an LDS slot: RoPE, Hadamard and the
// NVFP4 round trip of the group's query columns (exact in fp16), laid out as
// the B operands of QK^T: slot[t][c][lane] holds, for lane (c16, g4), dims
// 32*g4 + 8c .. +7 of column 16t + c16.  PACKED: columns 8-15 repeat
// columns 0-7.  Columns past the group are zero.  The rows of a tile are
// first written row-major to `qrow` (16 x 128 halves of LDS scratch), or,
// with several tiles, to the tile's own slot memory, which is then
// rewritten in operand order.
template <bool PACKED, int kPasses, bool MQ, int NT>
__device__ __forceinline__ void make_q_operands(QIn<kPasses, MQ>& in, int group, int rotary_dim,
                                                const float* __restrict__ rope_cos,
                                                const float* __restrict__ rope_sin, int hadamard,
                                                const SignMask& signs, _Float16* qrow,
                                                h8 (*slot)[4][q_entries<PACKED>()]) {
  const int lane = (int)threadIdx.x;
  const int g4 = lane >> 4, c16 = lane & 15;
  constexpr int kTilePasses = kPasses / NT;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
  // (rows staged in the slot itself when it holds them: several tiles, or
  // the up to 8 rows of a packed group)
  constexpr bool kInSlot = NT > 1 || PACKED;
  _Float16* rows = kInSlot ? reinterpret_cast<_Float16*>(&slot[t][0][0]) : qrow;
#pragma unroll
  for (int pass = kTilePasses * t; pass < kTilePasses * (t + 1); ++pass) {
    if (pass * 4 >= group) break;
    const int h = pass * 4 + g4;
    uint32_t codes, scode;
    if (MQ) {
      if (rotary_dim > 0)
        rope_coeffs_q<kGR>(c16, rotary_dim, rope_cos + (size_t)in.pos[pass] * (rotary_dim / 2),
                           rope_sin + (size_t)in.pos[pass] * (rotary_dim / 2), in.rc, in.rs);
      else
        in.rc[0] = in.rc[1] = in.rs[0] = in.rs[1] = u4{0u, 0u, 0u, 0u};
    }
    // the append kernel's row quantizer (the NVFP4 round trip of K rows)
    float x[8];
    q_unpack(in.w[pass], in.dtype, x);
    rowq::RopeLane rl;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      rl.cv[k] = __uint_as_float(in.rc[k / 4][k % 4]);
      rl.sv[k] = __uint_as_float(in.rs[k / 4][k % 4]);
    }
    const int hl = rotary_dim / 16;   // lanes per rotary half
    rl.first = c16 < hl;
    rl.in_rot = c16 < 2 * hl;
    rl.src = rl.in_rot ? (rl.first ? c16 + hl : c16 - hl) : c16;
    rowq::append_row16<kGR>(x, c16, rotary_dim > 0, rotary_dim, rl, hadamard != 0,
                            lane_signs(hadamard, signs, c16), hadamard == 2, codes, scode);
    // exact fp16 operands: E2M1 values times 2^8, then the E4M3 scale times
    // 2^-8 (the scale byte shifted left by 7 is its fp16 encoding)
    const h2 sc = bits_h2((scode << 7) | (scode << 23));
    h8 qv;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const h2 v = fp4x2(codes, b) * sc;
      qv[2 * b] = v[0];
      qv[2 * b + 1] = v[1];
    }
    if (h < group) *reinterpret_cast<h8*>(&rows[(h - 16 * t) * kHeadDim + 8 * c16]) = qv;
  }
  __syncthreads();
  const int qcol = PACKED ? (c16 & 7) : c16;
  h8 v[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    h8 z = {0, 0, 0, 0, 0, 0, 0, 0};
    v[c] = (16 * t + qcol < group) ? *reinterpret_cast<const h8*>(&rows[qcol * kHeadDim + 32 * g4 + 8 * c]) : z;
  }
  if (kInSlot) __syncthreads();   // every row read before the slot is rewritten
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (!PACKED) slot[t][c][lane] = v[c];
    else if (c16 < 8) slot[t][c][g4 * 8 + c16] = v[c];
  }
  // the zero entries (rows staged in the slot may have covered them)
  if (lane < 4) slot[t][lane][q_entries<PACKED>() - 1] = h8{0, 0, 0, 0, 0, 0, 0, 0};
  __syncthreads();
  }
}

// The current token of segment sg (token seq_lens[seq] - 1) quantized into
// its pool slot exactly as the append kernel does it: lanes 0-15 the K row
// (RoPE at q_positions[seq], Hadamard), lanes 16-31 the V row (quantized, or
// with `vf16` rounded to fp16); lanes 32-63 repeat the two rows (every lane
// takes part in the shuffles) and store nothing.
__device__ __forceinline__ void append_new_token(
    int sg, uint8_t* __restrict__ pool, int64_t num_pages, int hkv, int layer,
    const void* __restrict__ k_new, const void* __restrict__ v_new, int in_dtype,
    const int32_t* __restrict__ q_positions, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, int rotary_dim, int hadamard, const SignMask& signs,
    const int32_t* __restrict__ page_table, int pt_stride, const int32_t* __restrict__ seq_lens,
    float2 kv_inv, bool vf16) {
  const int lane = (int)threadIdx.x;
  const int c16 = lane & 15;
  const int which = (lane >> 4) & 1;   // 0 = K, 1 = V
  const int seq = sg / hkv, kvh = sg % hkv;
  float x[8];
  load8(which ? v_new : k_new, in_dtype, ((size_t)seq * hkv + kvh) * kHeadDim + 8 * c16, x);
  // the global scale divides the inputs (by the binary32 reciprocal)
  const float inv = which ? kv_inv.y : kv_inv.x;
#pragma unroll
  for (int k = 0; k < 8; ++k) x[k] *= inv;
  const int rot = which ? 0 : rotary_dim;
  const float* crow = nullptr;
  const float* srow = nullptr;
  if (rot > 0) {
    const int pos = q_positions[seq];
    crow = rope_cos + (size_t)pos * (rotary_dim / 2);
    srow = rope_sin + (size_t)pos * (rotary_dim / 2);
  }
  uint32_t codes, scode;
  quant_row16<kGR>(x, c16, rot, crow, srow, which ? false : (hadamard != 0),
              which ? 0u : lane_signs(hadamard, signs, c16), codes, scode);
  if (lane < 32) {
    const int tok = seq_lens[seq] - 1;
    const int page = page_table[(size_t)seq * pt_stride + tok / kPageSize];
    const uint32_t t = (uint32_t)(tok % kPageSize);
    uint8_t* blk = pool + (((size_t)layer * (size_t)num_pages + (size_t)page) * (size_t)hkv + kvh) *
                              (size_t)(vf16 ? kBlockBytesF16V : kBlockBytes);
    if (which && vf16) {
      // (V rows get neither RoPE nor the rotation: x still holds the inputs)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        *reinterpret_cast<uint16_t*>(blk + v16_off(t, (uint32_t)(8 * c16 + k))) = (uint16_t)f16_bits(x[k]);
    } else {
      *reinterpret_cast<uint32_t*>(blk + (which ? v_code_word_off(t, (uint32_t)c16)
                                                : k_code_word_off(t, (uint32_t)c16))) = codes;
      if ((c16 & 1) == 0)
        blk[(which ? kVScaleOff : (vf16 ? kKScaleOffF16V : kKScaleOff)) + 8 * t + c16 / 2] = (uint8_t)scode;
    }
  }
}

__device__ inline float row_ror8(float x) {
  // the value of lane (c16 + 8) % 16 of the same 16-lane row
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, true));
}

// Partial (m, l, acc) of the columns col0 .. col0 + 15 (those below
// `group`) to slot `slot`.  PAIRED: lanes c16 and c16 + 8 summed the
// weights of different tokens of the same column, so their sums add up.
template <bool PACKED, bool PAIRED = false>
__device__ __forceinline__ void write_partial(const f4 (&acc)[8], float m_ref, float l_run, int c16,
                                              int g4, int group, float* __restrict__ ws_acc,
                                              float2* __restrict__ ws_ml, size_t slot, int col0) {
  f4 o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    o[j] = acc[j];
    if (PACKED) {
      // column h += column h + 8 (high + low parts of the weights)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[j][i] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(acc[j][i]), 0x128, 0xF, 0xF, true));
    }
  }
  float l_tot = sum4lanes(l_run);
  if (PAIRED) l_tot += row_ror8(l_tot);
  const int col = col0 + c16;
  if (col < group) {
    // lane holds dims 32*g4 + 8i + j in o[j][i]
    float* dst = ws_acc + (slot * group + col) * kHeadDim + 32 * g4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      reinterpret_cast<float4*>(dst + 8 * i)[0] = make_float4(o[0][i], o[1][i], o[2][i], o[3][i]);
      reinterpret_cast<float4*>(dst + 8 * i)[1] = make_float4(o[4][i], o[5][i], o[6][i], o[7][i]);
    }
    if (g4 == 0) ws_ml[slot * group + col] = make_float2(m_ref, l_tot);
  }
}

// Where a finished segment's partial goes.
struct SegState {
  size_t slot;        // partial slot of the current segment (segment + wave)
};

// Online softmax of one unit for one column tile with the segment switch
// folded into its rare branch: when `sw` is set, the unit is the first of a
// new segment, so the finished segment's partial goes to slot `slot` and the
// running state restarts (reference -inf, so the rescale factor is 0).
template <bool MASKED, bool PACKED>
__device__ __forceinline__ void softmax_sw(const f4 (&S)[2], int g4, int c16, int nvalid,
                                           float c_log2, float lo_mask, f4 (&acc)[8], float& m_ref,
                                           float& l_run, h8& p0, h8& p1, bool sw, int group,
                                           float* __restrict__ ws_acc, float2* __restrict__ ws_ml,
                                           size_t slot, int cut, int col0) {
  // the lane's column sees the unit's first nvalid - cut tokens (cut > 0
  // only for the earlier of several new query tokens)
  if (MASKED) nvalid -= cut;
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (!MASKED || 16 * i + 4 * g4 + r < nvalid) mx = fmaxf(mx, S[i][r]);
  mx *= c_log2;
  if (sw || __builtin_amdgcn_ballot_w64(mx > m_ref + kMargin)) {
    if (sw) {
      write_partial<PACKED>(acc, m_ref, l_run, c16, g4, group, ws_acc, ws_ml, slot, col0);
      m_ref = -INFINITY;
      l_run = 0.0f;
    }
    const float m_new = fmaxf(m_ref, max4lanes(mx));
    // (a column with no valid score yet keeps -inf and zero sums, also right
    // after a segment switch; 2^(-inf - -inf) would make them NaN)
    const float alpha = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
    l_run *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    m_ref = m_new;
  }
  const float off = kOff - m_ref;
  float P[8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float e = __builtin_amdgcn_exp2f(fmaf(S[i][r], c_log2, off));
      if (MASKED && 16 * i + 4 * g4 + r >= nvalid) e = 0.0f;
      P[4 * i + r] = e;
      l_run += e;
    }
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    const float pa = P[2 * s2], pb = P[2 * s2 + 1];
    const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(pa, pb));
    h2 lo;
    if (PACKED) {
      // columns 8-15 (lo_mask 1) take the exact remainder, columns 0-7 the
      // truncated value itself (remainder of nothing subtracted)
      lo = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(fmaf(-lo_mask, (float)hi[0], pa),
                                                             fmaf(-lo_mask, (float)hi[1], pb)));
      p0[2 * s2] = lo[0];
      p0[2 * s2 + 1] = lo[1];
    } else {
      lo = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(sub_f16<false>(pa, hi), sub_f16<true>(pb, hi)));
      p0[2 * s2] = hi[0];
      p0[2 * s2 + 1] = hi[1];
      p1[2 * s2] = lo[0];
      p1[2 * s2 + 1] = lo[1];
    }
  }
}

// Softmax of one unit in the common case: every token valid, no segment
// switch.  Returns true, leaving everything untouched, when some score
// passes the reference by kMargin (the caller then takes the general path,
// which moves the reference and rescales); else turns the scores into the
// weight operands.  Having no rescale here keeps the accumulators free of
// any conditional update on the common path.
template <bool PACKED, int NT>
__device__ __forceinline__ bool softmax_fast(const f4 (&S)[NT][2], float c_log2, float lo_mask,
                                             const float (&m_ref)[NT], float (&l_run)[NT], h8 (&p0)[NT],
                                             h8 (&p1)[NT]) {
  bool over = false;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float mx = fmaxf(fmaxf(fmaxf(S[t][0][0], S[t][0][1]), fmaxf(S[t][0][2], S[t][0][3])),
                     fmaxf(fmaxf(S[t][1][0], S[t][1][1]), fmaxf(S[t][1][2], S[t][1][3])));
    mx *= c_log2;
    over = over || mx > m_ref[t] + kMargin;
  }
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(over) != 0, 0)) return true;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float off = kOff - m_ref[t];
    float P[8];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(S[t][i][r], c_log2, off));
        P[4 * i + r] = e;
        l_run[t] += e;
      }
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) {
      const float pa = P[2 * s2], pb = P[2 * s2 + 1];
      const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(pa, pb));
      h2 lo;
      if (PACKED) {
        lo = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(fmaf(-lo_mask, (float)hi[0], pa),
                                                               fmaf(-lo_mask, (float)hi[1], pb)));
        p0[t][2 * s2] = lo[0];
        p0[t][2 * s2 + 1] = lo[1];
      } else {
        lo = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(sub_f16<false>(pa, hi), sub_f16<true>(pb, hi)));
        p0[t][2 * s2] = hi[0];
        p0[t][2 * s2 + 1] = hi[1];
        p1[t][2 * s2] = lo[0];
        p1[t][2 * s2 + 1] = lo[1];
      }
    }
  }
  return false;
}

// Softmax of one unit for every column tile: unmasked when the unit's
// nvalid tokens cover the whole unit for every column (full_at = 32 + the
// largest cut), else masked.  A segment switch moves to the next slot once
// every tile's partial is written.
template <bool PACKED, int NT>
__device__ __forceinline__ void softmax_pick(int nvalid, int full_at, const f4 (&S)[NT][2], int g4,
                                             int c16, float c_log2, float lo_mask, f4 (&acc)[NT][8],
                                             float (&m_ref)[NT], float (&l_run)[NT], h8 (&p0)[NT],
                                             h8 (&p1)[NT], bool sw, int group,
                                             float* __restrict__ ws_acc, float2* __restrict__ ws_ml,
                                             SegState& st, const int (&cut)[NT]) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (nvalid >= full_at)
      softmax_sw<false, PACKED>(S[t], g4, c16, nvalid, c_log2, lo_mask, acc[t], m_ref[t], l_run[t], p0[t],
                                p1[t], sw, group, ws_acc, ws_ml, st.slot, cut[t], 16 * t);
    else
      softmax_sw<true, PACKED>(S[t], g4, c16, nvalid, c_log2, lo_mask, acc[t], m_ref[t], l_run[t], p0[t],
                               p1[t], sw, group, ws_acc, ws_ml, st.slot, cut[t], 16 * t);
  }
  if (sw) st.slot += 1;
}

// Softmax of a whole page (both 32-token units) at once, for groups of up
// to 8 query heads.  Their query operands repeat columns 0-7 in columns
// 8-15; QK^T of the page's first unit takes them with columns 8-15 zeroed,
// that of its second unit with columns 0-7 zeroed and accumulates onto the
// first, so lanes c16 < 8 hold unit 0's scores (token 16i + 4*g4 + r of the
// page in S[i][r]) and lanes c16 >= 8 unit 1's (token 32 + 16i + 4*g4 + r),
// and one pass of exponentials covers the page.  Lanes c16 and
// c16 ^ 8 belong to the same query head and keep the same reference.  The
// weight operands of the two PV steps then take the fp16 high part in
// columns 0-7 and the exact remainder in columns 8-15, the half that lives
// in the other lane of the pair brought over by a row rotation:
//   unit 0 (pa): c16 < 8 own high part, c16 >= 8 partner's remainder;
//   unit 1 (pb): c16 < 8 partner's high part, c16 >= 8 own remainder.
__device__ __forceinline__ void pair_operands(const float (&P)[8], bool upper, h8& pa, h8& pb) {
  u4 ua, ub;
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    const float x = P[2 * s2], y = P[2 * s2 + 1];
    const h2 hi = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(x, y));
    const h2 lo = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(fmaf(-1.0f, (float)hi[0], x),
                                                                   fmaf(-1.0f, (float)hi[1], y)));
    const uint32_t hb = __builtin_bit_cast(uint32_t, hi), lb = __builtin_bit_cast(uint32_t, lo);
    const uint32_t hr = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hb, 0x128, 0xF, 0xF, true);
    const uint32_t lr = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lb, 0x128, 0xF, 0xF, true);
    ua[s2] = upper ? lr : hb;
    ub[s2] = upper ? lb : hr;
  }
  pa = __builtin_bit_cast(h8, ua);
  pb = __builtin_bit_cast(h8, ub);
}

// Page softmax: tokens past `nvalid` (the page's valid tokens, less `cut`
// for the lane's column) are masked when MASKED, and `sw` starts a new
// segment (the finished one's partial goes to slot `slot` first).  The
// reference moves only when some score passes it by kMargin.
template <bool MASKED>
__device__ __forceinline__ void softmax_page(const f4 (&S)[2], int g4, int c16, int nvalid,
                                             float c_log2, f4 (&acc)[8], float& m_ref, float& l_run,
                                             h8& pa, h8& pb, bool sw, int group,
                                             float* __restrict__ ws_acc, float2* __restrict__ ws_ml,
                                             size_t slot, int cut) {
  const bool upper = c16 >= 8;
  const int nv = nvalid - (upper ? 32 : 0) - cut;
  float x[8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) x[4 * i + r] = S[i][r];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (!MASKED || 16 * i + 4 * g4 + r < nv) mx = fmaxf(mx, x[4 * i + r]);
  mx *= c_log2;
  if (sw || __builtin_amdgcn_ballot_w64(mx > m_ref + kMargin)) {
    if (sw) {
      write_partial<true, true>(acc, m_ref, l_run, c16, g4, group, ws_acc, ws_ml, slot, 0);
      m_ref = -INFINITY;
      l_run = 0.0f;
    }
    float mg = max4lanes(mx);
    mg = fmaxf(mg, row_ror8(mg));
    const float m_new = fmaxf(m_ref, mg);
    const float alpha = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
    l_run *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
    m_ref = m_new;
  }
  const float off = kOff - m_ref;
  float P[8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float e = __builtin_amdgcn_exp2f(fmaf(x[4 * i + r], c_log2, off));
      if (MASKED && 16 * i + 4 * g4 + r >= nv) e = 0.0f;
      P[4 * i + r] = e;
      l_run += e;
    }
  pair_operands(P, upper, pa, pb);
}

// Query-operand slots in LDS per wave: segment s of the range uses slot
// (s - first segment) % 3, enough for the (at most three) segments one trip
// of the page loop touches.
constexpr int kQSlots = 3;

// Stream-K decode.  All (sequence, kv head, page) work is laid out flat:
// segment g = seq * hkv + kvh holds that pair's pages, segments in order,
// each followed by kSegExtra units of no work.  With TU units in all and W =
// gridDim.x wavefronts, wave w takes the pages of units [w*TU/W,
// (w+1)*TU/W), so every wave gets the same amount of work (+-1 page), a
// segment end counting as kSegExtra pages, whatever the sequence lengths.  A
// range may start or end inside a segment and may cover several; the wave
// writes one partial per segment it touches, to slot g + w (distinct for
// every (segment, wave) pair).
//
// The wave walks its range as one stream of pages: two register sets, A for
// the range's even pages and B for its odd pages, so every load is issued
// two pages before its data is used, and the stream does not stop at a
// segment boundary.  Within the stream, a software pipeline over 32-token
// units: one straight-line block does QK^T of unit u+1 and PV of unit u,
// two independent streams of dequantization and MFMAs, then the softmax of
// unit u+1 turns its scores into the weights that the next block's PV uses.
// Loads are unconditional (past the range the buffer resource is empty and
// returns zeros without memory traffic) so the wait counts stay exact.
//
// Each lane of the wave describes one page of a 64-page window of the
// range: its pool block (page * hkv + kv head), its valid tokens, its page
// index inside its segment and its segment; the loop reads these with
// readlane, so no scalar loads sit on its path.
//
// NT column tiles of 16 (several new query tokens per sequence, up to 48
// columns) share every dequantized K and V operand: the page is read and
// dequantized once and feeds NT times the MFMAs and softmax work.  Those
// kernels hold NT sets of scores, weights and accumulators and run one
// wavefront per SIMD.
//
// VF16 (the fp16-V pool format, page-softmax kernels only): V tiles are
// loaded as fp16 operands, 16 KB a page, and go to the matrix instructions
// without dequantization.
template <bool PACKED, bool MQ, int NT, bool VF16 = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(NT > 1 ? 1 : 2, NT > 1 ? 1 : 2))) void decode_attn_splitk_kernel(
    uint8_t* __restrict__ pool, int64_t num_pages, int hkv, int layer, int n_seq, int n_q_heads,
    QCols qc, const void* __restrict__ q, const void* __restrict__ k_new,
    const void* __restrict__ v_new, int in_dtype, const int32_t* __restrict__ q_positions,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin, int rotary_dim,
    int hadamard, SignMask signs, const int32_t* __restrict__ page_table, int pt_stride,
    const int32_t* __restrict__ seq_lens, float c_log2, float* __restrict__ ws_acc,
    float2* __restrict__ ws_ml, float2 kv_inv) {
  __shared__ __attribute__((aligned(16))) u4 sc_lds[2][64];
  constexpr int kQE = q_entries<PACKED>();
  __shared__ __attribute__((aligned(16))) h8 q_lds[kQSlots][NT][4][kQE];
  __shared__ __attribute__((aligned(16))) _Float16 qrow[(NT > 1 || PACKED) ? 8 : 16 * kHeadDim];

  const int lane = (int)threadIdx.x;
  // the zero entry of every slot row
  if (lane < kQSlots * NT * 4) q_lds[lane / (NT * 4)][(lane / 4) % NT][lane % 4][kQE - 1] = h8{0, 0, 0, 0, 0, 0, 0, 0};
  const int g4 = lane >> 4;     // lane group
  const int c16 = lane & 15;    // column: query head for S/P/O, operand row for K/V
  const int group = qc.group;
  // Several new query tokens: the lane's column (its query token j) sees the
  // sequence up to token seq_len - n_qtok + j, i.e. `cut` tokens less than
  // the last one; a unit is full for every column only from `mcut` tokens
  // past its end on.
  int cut[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int col = 16 * t + (PACKED ? (c16 & 7) : c16);
    cut[t] = MQ ? max(qc.n_qtok - 1 - (qc.qtok0 + min(col, group - 1) / qc.heads), 0) : 0;
  }
  const int mcut = MQ ? qc.n_qtok - 1 - qc.qtok0 : 0;
  __builtin_amdgcn_s_setprio(3);
  const int64_t W = gridDim.x, w = blockIdx.x;
  // the sequences' offsets across the wavefront (kWalkSeqs + 1 up to
  // kScanSeqs of them), else walks over the lengths
  const bool scan = n_seq > kWalkSeqs && n_seq <= kScanSeqs;
  SeqScan sc;
  if (scan) seq_scan(seq_lens, n_seq, hkv, sc);
  int64_t TU;
  if (scan) {
    TU = sc.TU;
  } else {
    int64_t TP = 0;
    for (int s = 0; s < n_seq; ++s) TP += seq_pages(seq_lens, s);
    TU = TP * hkv + (int64_t)kSegExtra * n_seq * hkv;
  }
  // this wave's pages: those of its work units [w*TU/W, (w+1)*TU/W)
  const int64_t u_a = (w * TU) / W, u_b = ((w + 1) * TU) / W;
  const int64_t a = scan ? scan_page_of_unit(sc, u_a, n_seq) : page_of_unit(u_a, seq_lens, n_seq, hkv);
  const int64_t b = scan ? scan_page_of_unit(sc, u_b, n_seq) : page_of_unit(u_b, seq_lens, n_seq, hkv);
  if (a >= b) return;

  // segment holding page a: sequence, kv head, flat index of its first page
  int seq = 0;
  int64_t seq_base = 0;
  int64_t pg;
  if (scan) {
    seq = scan_seq_at(sc.p0, a, n_seq);
    seq_base = readlane64(scan_chunk(sc.p0, seq >> 6), seq & 63);
    pg = scan_pages(sc, seq);
  } else {
    pg = seq_pages(seq_lens, 0);
    while (a >= seq_base + hkv * pg) {
      seq_base += hkv * pg;
      ++seq;
      pg = seq_pages(seq_lens, seq);
    }
  }
  const int kvh0 = (int)((a - seq_base) / pg);
  const int seg0 = seq * hkv + kvh0;

  // ---- page window: lane i describes flat page a + wo + i of the range.
  // Pages of the range are counted from a in 32 bits (npg < 2^30, checked
  // on the host), so the loop's bookkeeping is scalar arithmetic.
  const int npg = (int)(b - a);
  int wo = 0;
  int w_blk, w_nv, w_j, w_sg;
  // the window's entries for lanes whose page x lies in sequence lseq, kv
  // head lkvh, whose segment starts at flat page lstart
  auto set_window = [&](int lseq, int lkvh, int64_t lstart, int64_t x) {
    const int j = (int)(x - lstart);
    w_blk = page_table[(size_t)lseq * pt_stride + j] * hkv + lkvh;
    // the sequence's length as loaded: the page's valid tokens are taken
    // where they are read (lanes past the range are never read)
    w_nv = seq_lens[lseq];
    w_j = j;
    w_sg = lseq * hkv + lkvh;
  };
  // the window at wo by a walk from the segment holding page a + wo (the
  // loop's reloads, and the first window past kScanSeqs sequences)
  auto load_window = [&](int wseq, int wkvh, int64_t wstart, int64_t wpg) {
    int lseq = wseq, lkvh = wkvh;
    int64_t lstart = wstart, lpg = wpg;
    const int64_t x = min(a + wo + lane, b - 1);
    while (x >= lstart + lpg) {
      lstart += lpg;
      if (++lkvh == hkv) {
        lkvh = 0;
        ++lseq;
        lpg = seq_pages(seq_lens, lseq);
      }
    }
    set_window(lseq, lkvh, lstart, x);
  };
  if (scan) {
    // the first window from the scan: each lane's sequence by search, its kv
    // head and page by division (kept out of the lambdas, so the scan's
    // registers are not addressed and die here)
    const int64_t x = min(a + lane, b - 1);
    const int lseq = scan_seq_of_page_lane(sc, x, n_seq);
    const int c = lseq >> 6;
    const int lpg = scan_shfl(sc.pg, c, lseq & 63, n_seq);
    const int64_t sb = scan_shfl(sc.p0, c, lseq & 63, n_seq);
    const uint32_t r = (uint32_t)(x - sb);   // < hkv * pages of one sequence
    const int lkvh = (int)(r / (uint32_t)lpg);
    set_window(lseq, lkvh, sb + (int64_t)lkvh * lpg, x);
  } else {
    load_window(seq, kvh0, seq_base + (int64_t)kvh0 * pg, pg);
  }

  // ---- the current token of every segment whose last page is in the range
  // goes into the cache here (only this wavefront reads that page), and its
  // stores land before that page's loads are issued.  A token whose page is
  // among the range's first two pages is written before any page load;
  // the others after the first two pages' loads are on their way, so the
  // wavefront does not start late.
  auto append_tokens = [&](bool first_pages) {
    bool any = false;
    int sq = seq, kv = kvh0;
    int64_t sstart = seq_base + (int64_t)kvh0 * pg, pgl = pg;
    while (sstart < b) {
      const int64_t last = sstart + pgl - 1;
      if (pgl > 0 && last >= a && last < b && (last <= a + 1) == first_pages) {
        append_new_token(sq * hkv + kv, pool, num_pages, hkv, layer, k_new, v_new, in_dtype,
                         q_positions, rope_cos, rope_sin, rotary_dim, hadamard, signs, page_table,
                         pt_stride, seq_lens, kv_inv, VF16);
        any = true;
      }
      sstart += pgl;
      if (++kv == hkv) {
        kv = 0;
        if (++sq >= n_seq) break;
        pgl = seq_pages(seq_lens, sq);
      }
    }
    return any;
  };
  if (k_new != nullptr && append_tokens(true)) {
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
  }


  static_assert(!VF16 || (PACKED && NT == 1 && !MQ), "fp16 V: page-softmax kernel of one query token only");
  constexpr int kBB = VF16 ? kBlockBytesF16V : kBlockBytes;   // block bytes
  constexpr int kKS = VF16 ? kKScaleOffF16V : kKScaleOff;     // K scales in a block
  const uint8_t* layer_base =
      pool + (size_t)layer * (size_t)num_pages * (size_t)hkv * (size_t)kBB;
  // buffer resource of page a + i of the range (empty past the range)
  auto rsrc_of = [&](int i) {
    const bool ok = i < npg;
    const int blk = __builtin_amdgcn_readlane(w_blk, (ok ? i : npg - 1) - wo);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(layer_base + (size_t)blk * kBB),
                                             0, ok ? kBB : 0, 0x00020000);
  };
  auto nvalid_of = [&](int i) {
    return i < npg ? __builtin_amdgcn_readlane(w_nv, i - wo) - kPageSize * __builtin_amdgcn_readlane(w_j, i - wo)
                   : 0;
  };
  // first page of a segment other than page a's
  auto starts_segment = [&](int i) {
    return i < npg && __builtin_amdgcn_readlane(w_j, i - wo) == 0;
  };

  // query inputs of the range's first segment, and of the second when the
  // range reaches it, loaded before any page: made later, at the switch,
  // their loads would wait for the pages in flight (the wait counter is in
  // order).  With several column tiles the inputs are too many registers to
  // hold through the first page loads: their operands are made here.
  constexpr int kPasses = PACKED ? 2 : 4 * NT;
  QIn<kPasses, MQ> qin, qin2;
  load_q_inputs<kPasses, MQ>(seg0, hkv, n_q_heads, qc, q, in_dtype, q_positions, rope_cos, rope_sin,
                         rotary_dim, qin);
  const bool two_segs = b > seq_base + (int64_t)(kvh0 + 1) * pg;
  if (NT > 1) {
    make_q_operands<PACKED, kPasses, MQ, NT>(qin, group, rotary_dim, rope_cos, rope_sin, hadamard, signs, qrow,
                                             q_lds[0]);
    if (two_segs) {
      load_q_inputs<kPasses, MQ>(seg0 + 1, hkv, n_q_heads, qc, q, in_dtype, q_positions, rope_cos,
                                 rope_sin, rotary_dim, qin2);
      make_q_operands<PACKED, kPasses, MQ, NT>(qin2, group, rotary_dim, rope_cos, rope_sin, hadamard, signs,
                                               qrow, q_lds[1]);
    }
  } else if (two_segs) {
    load_q_inputs<kPasses, MQ>(seg0 + 1, hkv, n_q_heads, qc, q, in_dtype, q_positions, rope_cos,
                           rope_sin, rotary_dim, qin2);
  }

  const int voff = 16 * lane;
  // Scale bytes are staged with their sign bits cleared.  Written scales are
  // positive, so nothing changes for them; stale bytes of slots past the
  // sequence end then still decode to finite values (an E4M3 byte shifted
  // left by 7 is an fp16 Inf or NaN only with bit 7 set), and their zero
  // weights zero them in the MFMAs.
  // lane-invariant LDS byte offsets of this lane's scales inside a staged page
  const int sk_off = 8 * c16 + 2 * g4;            // K scales of token c16, blocks 2g4, 2g4+1
  const int sv_off = 512 + 32 * g4 + (c16 >> 1);  // V scales of token 4*g4, block c16/2
  const float lo_mask = (PACKED && c16 >= 8) ? 1.0f : 0.0f;

  f4 acc[NT][8];
  float m_ref[NT], l_run[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[t][j] = f4{0.f, 0.f, 0.f, 0.f};
    m_ref[t] = -INFINITY;
    l_run[t] = 0.0f;
  }
  SegState st{(size_t)seg0 + (size_t)w};
  int q_ready = two_segs ? seg0 + 1 : seg0;   // last segment whose query operands are in LDS
  // query operands of a segment from its LDS slot
  // (entry e: the lane's own, or kQE - 1 for zero columns)
  auto q_of = [&](int sg, h8 (&qb)[NT][4], int e) {
    if (NT > 1) asm volatile("" ::: "memory");
    const int sl = (sg - seg0) % kQSlots;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int c = 0; c < 4; ++c) qb[t][c] = q_lds[sl][t][c][e];
  };
  // Page softmax (one-tile groups of up to 8 heads): a page's first unit is
  // scored with columns 8-15 zero, its second with columns 0-7 zero
  constexpr bool kPageSoftmax = PACKED && NT == 1;
  const int e_own = PACKED ? g4 * 8 + (c16 & 7) : lane;
  const int e_lo = (kPageSoftmax && c16 >= 8) ? kQE - 1 : e_own;
  const int e_hi = c16 >= 8 ? e_own : kQE - 1;
  auto seg_of = [&](int i) { return __builtin_amdgcn_readlane(w_sg, min(i, npg - 1) - wo); };

  // ---- prologue: loads of the range's first two pages; unit 0's scores and
  // weights; the loads left in flight and their order are those of the
  // loop's back edge, so the wait counts at the loop head are the same on
  // entry and on the back edge.
  u4 kA[4], vA[4], sA, kB[4], vB[4], sB;
  u4 vH[VF16 ? 16 : 1];   // fp16 V of a page: units 0 and 1, 8 dim tiles each
  if constexpr (kPageSoftmax) {
    // one register set, loads one page ahead: page a's scales, K and V
    const __amdgpu_buffer_rsrc_t r0 = rsrc_of(0);
    sA = ld16(r0, voff, kKS);
    kA[0] = ld16(r0, voff, 0);
    kA[1] = ld16(r0, voff, 1024);
    kA[2] = ld16(r0, voff, 2048);
    kA[3] = ld16(r0, voff, 3072);
    if constexpr (VF16) {
#pragma unroll
      for (int j = 0; j < 16; ++j) vH[j] = ld16(r0, voff, kVCodeOff + 1024 * j);
    } else {
      vA[0] = ld16(r0, voff, kVCodeOff);
      vA[1] = ld16(r0, voff, kVCodeOff + 1024);
      vA[2] = ld16(r0, voff, kVCodeOff + 2048);
      vA[3] = ld16(r0, voff, kVCodeOff + 3072);
    }
    __builtin_amdgcn_sched_barrier(0);
  } else {
    const __amdgpu_buffer_rsrc_t r0 = rsrc_of(0), r1 = rsrc_of(1);
    sA = ld16(r0, voff, kKScaleOff);
    kA[0] = ld16(r0, voff, 0);
    kA[1] = ld16(r0, voff, 1024);
    __builtin_amdgcn_sched_barrier(0);
    kA[2] = ld16(r0, voff, 2048);
    kA[3] = ld16(r0, voff, 3072);
    vA[0] = ld16(r0, voff, kVCodeOff);
    vA[1] = ld16(r0, voff, kVCodeOff + 1024);
    sB = ld16(r1, voff, kKScaleOff);
    kB[0] = ld16(r1, voff, 0);
    kB[1] = ld16(r1, voff, 1024);
    vA[2] = ld16(r0, voff, kVCodeOff + 2048);
    vA[3] = ld16(r0, voff, kVCodeOff + 3072);
    kB[2] = ld16(r1, voff, 2048);
    kB[3] = ld16(r1, voff, 3072);
    vB[0] = ld16(r1, voff, kVCodeOff);
    vB[1] = ld16(r1, voff, kVCodeOff + 1024);
    __builtin_amdgcn_sched_barrier(0);
  }
  // query operands of the first segment, and the later-page tokens, while
  // the first pages load
  const bool late_appends = k_new != nullptr && append_tokens(false);
  if (NT == 1) {
    make_q_operands<PACKED, kPasses, MQ, NT>(qin, group, rotary_dim, rope_cos, rope_sin, hadamard, signs, qrow,
                                             q_lds[0]);
    if (two_segs)
      make_q_operands<PACKED, kPasses, MQ, NT>(qin2, group, rotary_dim, rope_cos, rope_sin, hadamard, signs,
                                               qrow, q_lds[1]);
  }
  if (late_appends) {
    __builtin_amdgcn_s_waitcnt(0);   // before the next loads, which may read those pages
    asm volatile("" ::: "memory");
  }
  f4 S[NT][2];
  h8 pw0[NT], pw1[NT], qb[NT][4];
  if constexpr (kPageSoftmax) {
    // page a staged and scored (both units); its scales in buffer 0, then
    // page a+1's scales and K on their way
    const __amdgpu_buffer_rsrc_t r1 = rsrc_of(1);
    sc_lds[0][lane] = sA & 0x7F7F7F7Fu;
    sA = ld16(r1, voff, kKS);
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(&sc_lds[0][0]);
    q_of(seg0, qb, e_lo);
    qk_unit<NT>(kA[0], kA[1], sb + sk_off, qb, S);
    kA[0] = ld16(r1, voff, 0);
    kA[1] = ld16(r1, voff, 1024);
    q_of(seg0, qb, e_hi);
    qk_unit<NT, true>(kA[2], kA[3], sb + sk_off + 256, qb, S);
    kA[2] = ld16(r1, voff, 2048);
    kA[3] = ld16(r1, voff, 3072);
    __builtin_amdgcn_sched_barrier(0);
  } else {
  {
    const __amdgpu_buffer_rsrc_t r1 = rsrc_of(1), r2 = rsrc_of(2);
    sc_lds[0][lane] = sA & 0x7F7F7F7Fu;
    sA = ld16(r2, voff, kKScaleOff);
    q_of(seg0, qb, e_lo);
    qk_unit<NT>(kA[0], kA[1], reinterpret_cast<const uint8_t*>(&sc_lds[0][0]) + sk_off, qb, S);
    kA[0] = ld16(r2, voff, 0);
    kA[1] = ld16(r2, voff, 1024);
    vB[2] = ld16(r1, voff, kVCodeOff + 2048);
    vB[3] = ld16(r1, voff, kVCodeOff + 3072);
    __builtin_amdgcn_sched_barrier(0);
    // (one-tile groups of up to 8 heads take the softmax a page at a time,
    // in the loop: page a's first unit stays scored, not yet weighted)
    if (!kPageSoftmax)
      softmax_pick<PACKED, NT>(nvalid_of(0), 32 + mcut, S, g4, c16, c_log2, lo_mask, acc, m_ref, l_run,
                               pw0, pw1, false, group, ws_acc, ws_ml, st, cut);
  }

  }
  // ---- main loop, two pages (p in set A, p+1 in set B) per trip.  Page p
  // is staged in LDS buffer 0, page p+1 in buffer 1.
  const uint8_t* sb0 = reinterpret_cast<const uint8_t*>(&sc_lds[0][0]);
  const uint8_t* sb1 = reinterpret_cast<const uint8_t*>(&sc_lds[1][0]);
  // Issue priority by progress.  Two wavefronts share each SIMD and, at
  // equal priority, the older one is issued first, so it would finish its
  // (equal) range long before the younger one, which then runs alone at a
  // lower issue rate.  Dropping the priority as the range is worked off
  // (below 50 % done: 3, then 2, 1 from 75 %, 0 from 90 %) hands the issue
  // slots to whichever wavefront is behind.
  const int t50 = npg / 2, t75 = (int)(3 * (int64_t)npg / 4), t90 = (int)(9 * (int64_t)npg / 10);
  if constexpr (kPageSoftmax) {
  // One-tile groups of up to 8 heads: the softmax covers a page (two units)
  // at once, and a page is one block of the software pipeline, its loads
  // one page ahead in one register set: softmax of page p (its scores made
  // by the block before), PV of its two units, QK^T of page p+1's two units.
  // At the top of the block for page p: S[0] holds page p's scores (its
  // first unit in lanes c16 < 8, its second in lanes c16 >= 8); page p's
  // scales are staged in LDS buffer (p - a) % 2; the registers hold page
  // p's V codes and page p+1's K codes and scales, in flight.  pa/pb are
  // the weight operands of page p's two units.
  h8 pa, pb;
  int next_prio = t50;   // page index of the next priority step
  for (int i = 0; i < npg; ++i) {
    if (__builtin_expect(i >= next_prio, 0)) {
      const int lv = i >= t90 ? 3 : i >= t75 ? 2 : 1;
      if (lv == 1) __builtin_amdgcn_s_setprio(2);
      else if (lv == 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
      next_prio = lv == 1 ? t75 : lv == 2 ? t90 : npg;
    }
    if (min(i + 2, npg - 1) - wo >= 64) {   // ranges of more than 64 pages
      const int o = i - wo;
      const int sg = __builtin_amdgcn_readlane(w_sg, o);
      const int j = __builtin_amdgcn_readlane(w_j, o);
      wo = i;
      load_window(sg / hkv, sg % hkv, a + i - j, seq_pages(seq_lens, sg / hkv));
    }
    const __amdgpu_buffer_rsrc_t r1 = rsrc_of(i + 1), r2 = rsrc_of(i + 2);
    const int nv = nvalid_of(i);
    const bool sw = i > 0 && starts_segment(i);
    const int sg1 = seg_of(i + 1);
    // query operands of a segment that starts at page p+1 (rare)
    while (q_ready < sg1) {
      ++q_ready;
      QIn<kPasses, MQ> in;
      load_q_inputs<kPasses, MQ>(q_ready, hkv, n_q_heads, qc, q, in_dtype, q_positions, rope_cos,
                                 rope_sin, rotary_dim, in);
      make_q_operands<PACKED, kPasses, MQ, NT>(in, group, rotary_dim, rope_cos, rope_sin, hadamard, signs,
                                               qrow, q_lds[(q_ready - seg0) % kQSlots]);
    }
    const int cur = i & 1;
    const uint8_t* sb_cur = reinterpret_cast<const uint8_t*>(&sc_lds[cur][0]);
    const uint8_t* sb_nxt = reinterpret_cast<const uint8_t*>(&sc_lds[cur ^ 1][0]);
    // page p+1's scales staged, page p+2's on their way
    sc_lds[cur ^ 1][lane] = sA & 0x7F7F7F7Fu;
    sA = ld16(r2, voff, kKS);
    if (nv >= 64 + mcut)
      softmax_page<false>(S[0], g4, c16, nv, c_log2, acc[0], m_ref[0], l_run[0], pa, pb, sw, group, ws_acc,
                          ws_ml, st.slot, cut[0]);
    else
      softmax_page<true>(S[0], g4, c16, nv, c_log2, acc[0], m_ref[0], l_run[0], pa, pb, sw, group, ws_acc,
                         ws_ml, st.slot, cut[0]);
    if (sw) st.slot += 1;
    if constexpr (VF16) {
      if (nv < 64) mask_v16(vH, nv, g4);
      pv_unit_f16<PACKED, NT>(reinterpret_cast<const u4(&)[8]>(vH[0]), reinterpret_cast<const h8(&)[NT]>(pa),
                              pw1, acc);
#pragma unroll
      for (int j = 0; j < 8; ++j) vH[j] = ld16(r1, voff, kVCodeOff + 1024 * j);
      pv_unit_f16<PACKED, NT>(reinterpret_cast<const u4(&)[8]>(vH[8]), reinterpret_cast<const h8(&)[NT]>(pb),
                              pw1, acc);
#pragma unroll
      for (int j = 8; j < 16; ++j) vH[j] = ld16(r1, voff, kVCodeOff + 1024 * j);
    } else {
    pv_unit<PACKED, NT>(vA[0], vA[1], sb_cur + sv_off, reinterpret_cast<const h8(&)[NT]>(pa), pw1, acc);
    vA[0] = ld16(r1, voff, kVCodeOff);
    vA[1] = ld16(r1, voff, kVCodeOff + 1024);
    pv_unit<PACKED, NT>(vA[2], vA[3], sb_cur + sv_off + 256, reinterpret_cast<const h8(&)[NT]>(pb), pw1, acc);
    vA[2] = ld16(r1, voff, kVCodeOff + 2048);
    vA[3] = ld16(r1, voff, kVCodeOff + 3072);
    }
    q_of(sg1, qb, e_lo);
    qk_unit<NT>(kA[0], kA[1], sb_nxt + sk_off, qb, S);
    kA[0] = ld16(r2, voff, 0);
    kA[1] = ld16(r2, voff, 1024);
    q_of(sg1, qb, e_hi);
    qk_unit<NT, true>(kA[2], kA[3], sb_nxt + sk_off + 256, qb, S);
    kA[2] = ld16(r2, voff, 2048);
    kA[3] = ld16(r2, voff, 3072);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
    write_partial<PACKED, kPageSoftmax>(acc[t], m_ref[t], l_run[t], c16, g4, group, ws_acc, ws_ml, st.slot, 16 * t);
  return;
  } else {
  int next_prio = t50;
  for (int i = 0; i < npg; i += 2) {
    if (__builtin_expect(i >= next_prio, 0)) {
      const int lv = i >= t90 ? 3 : i >= t75 ? 2 : 1;
      if (lv == 1) __builtin_amdgcn_s_setprio(2);
      else if (lv == 2) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
      next_prio = lv == 1 ? t75 : lv == 2 ? t90 : npg;
    }
    if (min(i + 4, npg - 1) - wo >= 64) {   // ranges of more than 64 pages
      const int o = i - wo;
      const int sg = __builtin_amdgcn_readlane(w_sg, o);
      const int j = __builtin_amdgcn_readlane(w_j, o);
      wo = i;
      load_window(sg / hkv, sg % hkv, a + i - j, seq_pages(seq_lens, sg / hkv));
    }
    const __amdgpu_buffer_rsrc_t r2 = rsrc_of(i + 2), r3 = rsrc_of(i + 3), r4 = rsrc_of(i + 4);
    const int nv0 = nvalid_of(i), nv1 = nvalid_of(i + 1), nv2 = nvalid_of(i + 2);
    const bool sw1 = starts_segment(i + 1), sw2 = starts_segment(i + 2);
    const int sg0 = seg_of(i), sg1 = seg_of(i + 1), sg2 = seg_of(i + 2);
    // query operands of segments that start in this trip (rare: a range
    // crosses few segment boundaries)
    while (q_ready < sg2) {
      ++q_ready;
      QIn<kPasses, MQ> in;
      load_q_inputs<kPasses, MQ>(q_ready, hkv, n_q_heads, qc, q, in_dtype, q_positions, rope_cos,
                             rope_sin, rotary_dim, in);
      make_q_operands<PACKED, kPasses, MQ, NT>(in, group, rotary_dim, rope_cos, rope_sin, hadamard, signs, qrow,
                                               q_lds[(q_ready - seg0) % kQSlots]);
    }

    // The four blocks of a trip: each does QK^T of one unit and PV of the
    // unit before it, and refills the registers it consumed with the page
    // two ahead.
    auto blk1 = [&]() {   // page p: tokens 32..63 scored, 0..31 accumulated
      q_of(sg0, qb, lane);
      qk_unit<NT>(kA[2], kA[3], sb0 + sk_off + 256, qb, S);
      kA[2] = ld16(r2, voff, 2048);
      kA[3] = ld16(r2, voff, 3072);
      pv_unit<PACKED, NT>(vA[0], vA[1], sb0 + sv_off, pw0, pw1, acc);
      vA[0] = ld16(r2, voff, kVCodeOff);
      vA[1] = ld16(r2, voff, kVCodeOff + 1024);
    };
    auto blk2 = [&]() {   // page p+1 staged; its 0..31 scored, page p's 32..63 accumulated
      sc_lds[1][lane] = sB & 0x7F7F7F7Fu;
      sB = ld16(r3, voff, kKScaleOff);
      q_of(sg1, qb, lane);
      qk_unit<NT>(kB[0], kB[1], sb1 + sk_off, qb, S);
      kB[0] = ld16(r3, voff, 0);
      kB[1] = ld16(r3, voff, 1024);
      pv_unit<PACKED, NT>(vA[2], vA[3], sb0 + sv_off + 256, pw0, pw1, acc);
      vA[2] = ld16(r2, voff, kVCodeOff + 2048);
      vA[3] = ld16(r2, voff, kVCodeOff + 3072);
    };
    auto blk3 = [&]() {   // page p+1: tokens 32..63 scored, 0..31 accumulated
      q_of(sg1, qb, lane);
      qk_unit<NT>(kB[2], kB[3], sb1 + sk_off + 256, qb, S);
      kB[2] = ld16(r3, voff, 2048);
      kB[3] = ld16(r3, voff, 3072);
      pv_unit<PACKED, NT>(vB[0], vB[1], sb1 + sv_off, pw0, pw1, acc);
      vB[0] = ld16(r3, voff, kVCodeOff);
      vB[1] = ld16(r3, voff, kVCodeOff + 1024);
    };
    auto blk4 = [&]() {   // page p+2 staged; its 0..31 scored, page p+1's 32..63 accumulated
      sc_lds[0][lane] = sA & 0x7F7F7F7Fu;
      sA = ld16(r4, voff, kKScaleOff);
      q_of(sg2, qb, lane);
      qk_unit<NT>(kA[0], kA[1], sb0 + sk_off, qb, S);
      kA[0] = ld16(r4, voff, 0);
      kA[1] = ld16(r4, voff, 1024);
      pv_unit<PACKED, NT>(vB[2], vB[3], sb1 + sv_off + 256, pw0, pw1, acc);
      vB[2] = ld16(r3, voff, kVCodeOff + 2048);
      vB[3] = ld16(r3, voff, kVCodeOff + 3072);
    };

    // Common trips (every unit full, no segment switch) take a path whose
    // softmax has no rescale branch; the first unit that needs one sends
    // the rest of the trip to the general path below, which picks up at
    // that unit.  Either way the loads go out in the same order.
    const bool regular =
        !sw1 && !sw2 && nv0 >= 64 + mcut && nv1 >= 64 + mcut && nv2 >= 32 + mcut && i + 1 < npg;
    int bail = 0;
    if (__builtin_expect(regular, 1)) {
      blk1();
      if (softmax_fast<PACKED, NT>(S, c_log2, lo_mask, m_ref, l_run, pw0, pw1)) { bail = 1; goto general; }
      blk2();
      if (softmax_fast<PACKED, NT>(S, c_log2, lo_mask, m_ref, l_run, pw0, pw1)) { bail = 2; goto general; }
      blk3();
      if (softmax_fast<PACKED, NT>(S, c_log2, lo_mask, m_ref, l_run, pw0, pw1)) { bail = 3; goto general; }
      blk4();
      if (softmax_fast<PACKED, NT>(S, c_log2, lo_mask, m_ref, l_run, pw0, pw1)) { bail = 4; goto general; }
      continue;
    }
  general:
    if (bail < 1) blk1();
    if (bail <= 1)
      softmax_pick<PACKED, NT>(nv0 - 32, 32 + mcut, S, g4, c16, c_log2, lo_mask, acc, m_ref, l_run,
                                  pw0, pw1, false, group, ws_acc, ws_ml, st, cut);
    if (bail < 2) blk2();
    if (bail <= 2)
      softmax_pick<PACKED, NT>(nv1, 32 + mcut, S, g4, c16, c_log2, lo_mask, acc, m_ref, l_run, pw0,
                                  pw1, sw1, group, ws_acc, ws_ml, st, cut);
    if (i + 1 >= npg) break;
    if (bail < 3) blk3();
    if (bail <= 3)
      softmax_pick<PACKED, NT>(nv1 - 32, 32 + mcut, S, g4, c16, c_log2, lo_mask, acc, m_ref, l_run,
                                  pw0, pw1, false, group, ws_acc, ws_ml, st, cut);
    if (bail < 4) blk4();
    softmax_pick<PACKED, NT>(nv2, 32 + mcut, S, g4, c16, c_log2, lo_mask, acc, m_ref, l_run, pw0,
                                pw1, sw2, group, ws_acc, ws_ml, st, cut);
  }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
    write_partial<PACKED>(acc[t], m_ref[t], l_run[t], c16, g4, group, ws_acc, ws_ml, st.slot, 16 * t);
}

#if !NVFP4KV_DECODE_GENERAL_ROPE
// Combine the partials of one (sequence, query head) for 32 output dims:
// 256 threads = 32 dims x 8 groups that stride over the pieces.  The pieces
// of segment g come from waves w_first .. w_last, found with the same flat
// indexing as the decode kernel; waves with an empty range (more waves than
// pages) wrote nothing and are skipped.
// DPT consecutive output dims of a piece's accumulator row (16-byte loads
// for 4).
template <int DPT>
__device__ __forceinline__ void load_dims(const float* __restrict__ p, float (&x)[DPT]) {
  if constexpr (DPT == 4) {
    const f4 v = *reinterpret_cast<const f4*>(p);
    x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
  } else {
    x[0] = *p;
  }
}

// Combine of a segment's pieces, at most 8 * NU of them, by a block of 256
// threads (thread: output dims col .. col + DPT - 1 of pieces j, j + 8, ...,
// j + 8 (NU - 1), j = tid / 32).  Each piece's (m, l) is requested first,
// then the accumulator entries, so the maximum and the weights are made
// while those are in flight.  Loads use indices clamped into the segment and
// the values past it get weight 0 (conditional loads became branches with
// waits between them).  Adds the thread's share to `acc` and `L`.
template <int NU, int DPT>
__device__ __forceinline__ void reduce_few(const float* __restrict__ ws_acc, const float2* __restrict__ ws_ml,
                                           size_t g, int64_t w0, int np, int group, int h, int col, int tid,
                                           int64_t TU, int64_t W, float* red_m, float* wts, float (&acc)[DPT],
                                           float& L) {
  constexpr int NP = 8 * NU;               // pieces covered
  constexpr int MLP = (NP + 255) / 256;    // (m, l) pairs per thread: pieces tid + 256k
  const int j = tid >> 5;
  float2 mlr[MLP];
  bool written[MLP];
#pragma unroll
  for (int k = 0; k < MLP; ++k) {
    const int p = tid + 256 * k;
    const int64_t w = w0 + p;
    // with at least as many units as wavefronts no range is empty
    written[k] = p < np && (TU >= W || (w * TU) / W != ((w + 1) * TU) / W);
    mlr[k] = ws_ml[(g + w0 + min(p, np - 1)) * group + h];
  }
  float a[NU][DPT];
#pragma unroll
  for (int u = 0; u < NU; ++u)
    load_dims<DPT>(ws_acc + ((g + w0 + min(j + 8 * u, np - 1)) * group + h) * kHeadDim + col, a[u]);
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < MLP; ++k) M = written[k] ? fmaxf(M, mlr[k].x) : M;
  for (int o = 16; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 32));
  if ((tid & 31) == 0) red_m[tid >> 5] = M;
  __syncthreads();
  M = red_m[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) M = fmaxf(M, red_m[i]);
  // weights by piece group: piece j + 8u at NU j + u, read back as vectors
#pragma unroll
  for (int k = 0; k < MLP; ++k) {
    const int p = tid + 256 * k;
    // (an unwritten slot's l may be anything: it is not multiplied either)
    const float wt = written[k] ? exp2f(mlr[k].x - M) : 0.0f;
    L += written[k] ? wt * mlr[k].y : 0.0f;
    if (p < NP) wts[NU * (p & 7) + (p >> 3)] = wt;
  }
  __syncthreads();
  // a piece of weight 0 adds nothing; its slot may never have been written
  // (a wavefront with an empty range), so it is not multiplied
  if constexpr (NU % 4 == 0) {
    const f4* wj = reinterpret_cast<const f4*>(wts + NU * j);
#pragma unroll
    for (int q = 0; q < NU / 4; ++q) {
      const f4 x = wj[q];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int d = 0; d < DPT; ++d) acc[d] += x[e] != 0.0f ? x[e] * a[4 * q + e][d] : 0.0f;
    }
  } else {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const float x = wts[NU * j + u];
#pragma unroll
      for (int d = 0; d < DPT; ++d) acc[d] += x != 0.0f ? x * a[u][d] : 0.0f;
    }
  }
}

// DPT output dims per thread: 1 (blocks of 32 dims, four per column) or 4
// (one block per column, 16-byte loads: a quarter of the blocks and of the
// load instructions, for launches with many columns).
template <int DPT>
__global__ __launch_bounds__(256) void decode_reduce_kernel(
    const float* __restrict__ ws_acc, const float2* __restrict__ ws_ml,
    const int32_t* __restrict__ seq_lens, int n_seq, int hkv, QCols qc, int n_q_heads, int64_t W,
    float v_scale, float* __restrict__ out) {
  const int group = qc.group;
  const int hq_idx = (int)blockIdx.x;     // column over all kv heads: kvh * group + c
  const int seq = (int)blockIdx.y;
  const int d0 = 32 * DPT * (int)blockIdx.z;   // first output dim of this block
  const int tid = (int)threadIdx.x;
  const int dd = tid & 31, j = tid >> 5;  // dim within the chunk, piece group
  const int kvh = hq_idx / group, h = hq_idx % group;
  // work units (pages plus kSegExtra per segment, as the decode kernel
  // splits them) before this segment and in all.  Up to 16 sequences: the
  // lengths through the scalar cache, 8 independent loads per wait (a
  // dependent load per sequence took a round trip each); more are read by
  // the block's threads side by side and summed across the block (with
  // thousands of blocks, scalar loads of every length from every wavefront
  // queued: 64 sequences, 6.3 against 1.7 us)
  __shared__ int64_t red_u[2][8];
  int64_t TU = 0, seq_base = 0, pg = 0;
  if (n_seq <= 16) {
    // at most 16 x (2^25 + 5) units: the sums fit in 32 unsigned bits
    uint32_t tu = 0, before = 0;
#pragma unroll
    for (int g8 = 0; g8 < 2; ++g8) {
      const int base = 8 * g8;
      if (base < n_seq) {
        int v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = seq_lens[min(base + i, n_seq - 1)];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int sq = base + i;
          const int pgi = (v[i] + kPageSize - 1) / kPageSize;
          const uint32_t u = sq < n_seq ? (uint32_t)(pgi + kSegExtra) : 0u;
          tu += u;
          before += sq < seq ? u : 0u;
          pg = sq == seq ? pgi : pg;
        }
      }
    }
    TU = tu;
    seq_base = before;
  } else {
    int64_t tu = 0, before = 0;
    for (int s = tid; s < n_seq; s += 256) {
      const int64_t u = seq_pages(seq_lens, s) + kSegExtra;
      tu += u;
      before += s < seq ? u : 0;
    }
    for (int o = 32; o > 0; o >>= 1) {
      tu += __shfl_xor(tu, o, 64);
      before += __shfl_xor(before, o, 64);
    }
    if ((tid & 63) == 0) {
      red_u[0][tid >> 6] = tu;
      red_u[1][tid >> 6] = before;
    }
    __syncthreads();
    TU = red_u[0][0] + red_u[0][1] + red_u[0][2] + red_u[0][3];
    seq_base = red_u[1][0] + red_u[1][1] + red_u[1][2] + red_u[1][3];
    pg = seq_pages(seq_lens, seq);
  }
  TU *= hkv;
  seq_base *= hkv;
  const int64_t S = seq_base + kvh * (pg + kSegExtra), E = S + pg;   // the segment's page units
  const int64_t w0 = wave_of(S, TU, W), w1 = wave_of(E - 1, TU, W);
  const size_t g = (size_t)seq * hkv + kvh;

  constexpr int kChunk = 1024;             // pieces whose weights are staged at once
  __shared__ float red_m[8];
  __shared__ __attribute__((aligned(16))) float red_o[8][32 * DPT];
  __shared__ float red_l[8];
  __shared__ __attribute__((aligned(16))) float wts[kChunk];
  float L = 0.0f, acc[DPT];
#pragma unroll
  for (int d = 0; d < DPT; ++d) acc[d] = 0.0f;
  const int col = d0 + DPT * dd;           // the thread's first output dim
  const int64_t np = w1 - w0 + 1;          // pieces of the segment
  // One round of loads up to 512 pieces with one dim per thread, 256 with
  // four (the accumulator entries held at once); past that, or for an empty
  // segment (no length of at least one token, which the interface requires,
  // gives one; the clamped loads need a piece), the staged path.
  if (np >= 1 && np <= (DPT == 1 ? 512 : 256)) {
    const int n = (int)np;
    if (n <= 8) {
      reduce_few<1, DPT>(ws_acc, ws_ml, g, w0, n, group, h, col, tid, TU, W, red_m, wts, acc, L);
    } else if (n <= 32) {
      reduce_few<4, DPT>(ws_acc, ws_ml, g, w0, n, group, h, col, tid, TU, W, red_m, wts, acc, L);
    } else if (n <= 64) {
      reduce_few<8, DPT>(ws_acc, ws_ml, g, w0, n, group, h, col, tid, TU, W, red_m, wts, acc, L);
    } else if (n <= 256) {
      reduce_few<32, DPT>(ws_acc, ws_ml, g, w0, n, group, h, col, tid, TU, W, red_m, wts, acc, L);
    } else {
      if constexpr (DPT == 1) reduce_few<64, 1>(ws_acc, ws_ml, g, w0, n, group, h, col, tid, TU, W, red_m, wts, acc, L);
    }
  } else {
  // ---- running max over all pieces
  float M = -INFINITY;
  for (int64_t w = w0 + tid; w <= w1; w += 256) {
    if (TU < W && (w * TU) / W == ((w + 1) * TU) / W) continue;
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
  for (int64_t c0 = w0; c0 <= w1; c0 += kChunk) {
    const int n = (int)((w1 - c0 + 1) < kChunk ? (w1 - c0 + 1) : kChunk);
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const int64_t w = c0 + i;
      float wt = 0.0f;
      if (TU >= W || (w * TU) / W != ((w + 1) * TU) / W) {
        const float2 ml = ws_ml[(g + w) * group + h];
        wt = exp2f(ml.x - M);
        L += wt * ml.y;
      }
      wts[i] = wt;
    }
    __syncthreads();
    for (int i = j; i < n; i += 128) {
      float a[16][DPT];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int iu = i + 8 * u < n ? i + 8 * u : i;
        load_dims<DPT>(ws_acc + ((g + c0 + iu) * group + h) * kHeadDim + col, a[u]);
      }
      // a piece of weight 0 adds nothing; its slot may never have been
      // written (a wavefront with an empty range), so it is not multiplied
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (i + 8 * u < n && wts[i + 8 * u] != 0.0f)
#pragma unroll
          for (int d = 0; d < DPT; ++d) acc[d] += wts[i + 8 * u] * a[u][d];
    }
  }
  }
  // L was summed per thread over its pieces; combine across the block
  for (int o = 16; o > 0; o >>= 1) L += __shfl_xor(L, o, 32);
#pragma unroll
  for (int d = 0; d < DPT; ++d) red_o[j][DPT * dd + d] = acc[d];
  if (dd == 0) red_l[j] = L;
  __syncthreads();
  if (j == 0) {
    float o[DPT], l = 0.0f;
#pragma unroll
    for (int d = 0; d < DPT; ++d) o[d] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int d = 0; d < DPT; ++d) o[d] += red_o[i][DPT * dd + d];
      l += red_l[i];
    }
    // column h of kv head kvh: head h % heads of query token qtok0 + h / heads
    const int tok = qc.qtok0 + h / qc.heads;
    float* dst = out + (((size_t)seq * qc.n_qtok + tok) * n_q_heads + (size_t)kvh * qc.heads + h % qc.heads) *
                           kHeadDim + col;
    // V's global scale: stored V values are V / v_scale
#pragma unroll
    for (int d = 0; d < DPT; ++d) dst[d] = o[d] * v_scale / l;
  }
}

#endif  // !NVFP4KV_DECODE_GENERAL_ROPE

}  // namespace

#if NVFP4KV_DECODE_GENERAL_ROPE
#define NVFP4KV_SPLITS_FN launch_decode_splits_gr
#else
#define NVFP4KV_SPLITS_FN launch_decode_splits
#endif

hipError_t NVFP4KV_SPLITS_FN(const LaunchPool& P, int layer, int n_seq, int n_q_heads,
                                const void* q, const void* k_new, const void* v_new, int in_dtype,
                                const int32_t* q_positions, const float* rope_cos,
                                const float* rope_sin, const int32_t* page_table,
                                int page_table_stride, const int32_t* seq_lens, float sm_scale,
                                void* workspace, const DecodePlan& plan, const QTokens& qt,
                                hipStream_t stream) {
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  float* ws_acc = reinterpret_cast<float*>(ws);
  float2* ws_ml = reinterpret_cast<float2*>(ws + ws_ml_offset(n_seq, P.hkv, plan));
  // K's global scale enters every score as a factor
  const float c_log2 = sm_scale * P.k_scale * 1.4426950408889634f;
  const QCols qc{plan.group, qt.heads, qt.n_qtok, qt.qtok0};
  const bool packed = plan.group <= 8, mq = qt.n_qtok > 1;
  const int nt = decode_column_tiles(plan.group);
  if (P.v_format != 0 && (!packed || mq)) return hipErrorInvalidValue;   // refused by the C ABI before
  auto kern = P.v_format != 0 ? decode_attn_splitk_kernel<true, false, 1, true>
              : nt == 3   ? decode_attn_splitk_kernel<false, true, 3>
              : nt == 2 ? decode_attn_splitk_kernel<false, true, 2>
              : packed  ? (mq ? decode_attn_splitk_kernel<true, true, 1> : decode_attn_splitk_kernel<true, false, 1>)
                        : (mq ? decode_attn_splitk_kernel<false, true, 1> : decode_attn_splitk_kernel<false, false, 1>);
  hipLaunchKernelGGL(kern, dim3(plan.n_waves), dim3(64), 0, stream, P.base, P.num_pages, P.hkv,
                     layer, n_seq, n_q_heads, qc, q, k_new, v_new, in_dtype, q_positions,
                     rope_cos, rope_sin, P.rotary_dim, P.hadamard, P.signs, page_table, page_table_stride,
                     seq_lens, c_log2, ws_acc, ws_ml, make_float2(P.k_inv, P.v_inv));
  return hipGetLastError();
}

#if !NVFP4KV_DECODE_GENERAL_ROPE
hipError_t launch_decode_reduce(int hkv, int n_seq, int n_q_heads, const int32_t* seq_lens,
                                float* out, const void* workspace, const DecodePlan& plan,
                                const QTokens& qt, float v_scale, hipStream_t stream) {
  const float* ws_acc = reinterpret_cast<const float*>(workspace);
  const float2* ws_ml = reinterpret_cast<const float2*>(reinterpret_cast<const uint8_t*>(workspace) +
                                                        ws_ml_offset(n_seq, hkv, plan));
  const QCols qc{plan.group, qt.heads, qt.n_qtok, qt.qtok0};
  // four blocks of 32 dims per column; with 1024 such blocks or more, one
  // block of 4 dims per thread per column instead
  const int64_t blocks = (int64_t)hkv * plan.group * n_seq * (kHeadDim / 32);
  if (blocks >= 1024)
    hipLaunchKernelGGL(decode_reduce_kernel<4>, dim3(hkv * plan.group, n_seq, kHeadDim / 128), dim3(256), 0,
                       stream, ws_acc, ws_ml, seq_lens, n_seq, hkv, qc, n_q_heads,
                       (int64_t)plan.n_waves, v_scale, out);
  else
    hipLaunchKernelGGL(decode_reduce_kernel<1>, dim3(hkv * plan.group, n_seq, kHeadDim / 32), dim3(256), 0,
                       stream, ws_acc, ws_ml, seq_lens, n_seq, hkv, qc, n_q_heads,
                       (int64_t)plan.n_waves, v_scale, out);
  return hipGetLastError();
}

// Workspace of the allocation-free decode entry point: every call on a GPU
// uses that GPU's copy, which keeps the last call's contents (the decode
// kernels need none of it cleared: the reduce reads only slots written by the
// same call).  Calls that overlap on one GPU race on it.
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

hipError_t static_workspace(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // with `dev` current: the address of this device's copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int decode_waves_per_cu(int nt, bool packed, bool vf16) {
  int lo = 1 << 30;
  if (vf16) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks, reinterpret_cast<const void*>(decode_attn_splitk_kernel<true, false, 1, true>), 64, 0) !=
        hipSuccess)
      return 0;
    return blocks;
  }
  const void* one_packed[2] = {reinterpret_cast<const void*>(decode_attn_splitk_kernel<true, false, 1>),
                               reinterpret_cast<const void*>(decode_attn_splitk_kernel<true, true, 1>)};
  const void* one[2] = {reinterpret_cast<const void*>(decode_attn_splitk_kernel<false, false, 1>),
                        reinterpret_cast<const void*>(decode_attn_splitk_kernel<false, true, 1>)};
  const void* two[1] = {reinterpret_cast<const void*>(decode_attn_splitk_kernel<false, true, 2>)};
  const void* three[1] = {reinterpret_cast<const void*>(decode_attn_splitk_kernel<false, true, 3>)};
  const int n = nt == 3 || nt == 2 ? 1 : 2;
  const void* const* kernels = nt == 3 ? three : nt == 2 ? two : packed ? one_packed : one;
  for (int i = 0; i < n; ++i) {
    const void* k = kernels[i];
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k, 64, 0) != hipSuccess) return 0;
    lo = blocks < lo ? blocks : lo;
  }
  return lo;
}

#endif  // !NVFP4KV_DECODE_GENERAL_ROPE

}  // namespace nvfp4kv
