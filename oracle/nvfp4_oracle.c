/*
 * CPU oracle for attention over a 4-bit NVFP4 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, and it shares no
 * code, header, table or constant generator with that path.
 *
 * Source of the method: the release post of the gzenz/ninfer fork
 * (prismix.dev news item 833001997676), section "NVFP4 KV cache (from
 * scratch)" and section "YaRN context extension".  In what follows that page
 * is called "the release post".  The post fixes:
 *   - K and V are stored as 4-bit NVFP4: E2M1 elements with hardware E4M3
 *     block scales; Q is quantized to NVFP4 as well (bullet 1);
 *   - K and Q are rotated by a Hadamard transform before quantization, V is
 *     not rotated (bullet 2);
 *   - the current token's K/V are quantized in place during decode (bullet 3);
 *   - KV scales are stored row-major, unswizzled (bullet 4);
 *   - 144 bytes per token per KV head (the "Result" line);
 *   - RoPE with theta 1e7 on 25 % of the dims, extended by linear position
 *     scaling (section "YaRN context extension").
 * Block size 16, head_dim 128 and the 128-point transform are the readings
 * that make 144 bytes come out: 2 x (64 code bytes + 8 scale bytes).
 *
 * Precision.  Attention is computed in double precision.  The steps before
 * quantization (RoPE, Hadamard) decide integer codes, so they are carried out
 * in IEEE binary32 with one rounding per operation and no fused multiply-add,
 * in the order written below; the device path takes the same decisions in the
 * same precision.  Build with -ffp-contract=off -fno-fast-math.
 *
 * Parity pins (tests/test_oracle_*.py) tie every function here to something
 * other than itself: library routines (scipy's Hadamard matrix, PyTorch's
 * float8_e4m3fn conversion), exact-fraction brute force, closed forms and
 * invariants.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_D 128         /* head dimension */
#define ORC_BLOCK 16      /* elements sharing one E4M3 scale */
#define ORC_NBLK 8        /* blocks per row */
#define ORC_PAGE 64       /* tokens per page */
#define ORC_ROW_CODE 64   /* code bytes per row (128 x 4 bit) */

/* Threads of the OpenMP loops below (timing only; results do not depend on
 * the thread count). */
void orc_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
}

int orc_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* E4M3 (OCP 8-bit float, "FN" variant): 1 sign, 4 exponent (bias 7), 3
 * mantissa bits, no infinities, 0x7F and 0xFF are NaN, largest finite 448.
 * Release post, NVFP4 section, bullet 1 ("E4M3 block scales"). */
double orc_e4m3_value(int code)
{
    code &= 0xFF;
    int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);               /* subnormal: m * 2^-9 */
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* Block scale for a block whose largest magnitude is amax: the E4M3 value
 * nearest to amax/6 (6 is the largest E2M1 magnitude), ties to the even code,
 * saturating at 448.  Found by brute force over the 127 finite non-negative
 * codes.  Distances are measured as |amax - 6*v|, i.e. scaled by 6, so that
 * no division is rounded; for amax <= 6*448 every distance that can decide
 * the choice is exact in double (amax has 24 significant bits, 6*v at most
 * 6).  Larger amax saturates to 448 (code 0x7E). */
int orc_e4m3_scale_code(float amax)
{
    double a = (double)amax;
    if (!(a >= 0.0)) return 0;                    /* not reached for finite input */
    if (a >= 6.0 * 448.0) return 0x7E;
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 127; ++c) {
        double d = fabs(a - 6.0 * orc_e4m3_value(c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = c;
        }
    }
    return best;
}

/* E2M1 (4-bit float): 1 sign, 2 exponent, 1 mantissa bit; magnitudes
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6.  Release post, NVFP4 section, bullet 1. */
double orc_e2m1_value(int nibble)
{
    static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    double v = mag[nibble & 7];
    return (nibble & 8) ? -v : v;
}

/* E2M1 code of element y in a block with scale s (an E4M3 value >= 0): the
 * magnitude whose multiple of s is nearest to |y|, ties to the even code,
 * saturating at 6; the sign bit is the sign bit of y.  A zero scale gives
 * magnitude 0.  |y| >= 6 s takes the largest magnitude directly (it is the
 * nearest); below that, the distances |(|y|) - v*s| that can decide are
 * exact in double (|y| has 24 significant bits and is below 6 s, v*s has at
 * most 6), and a |y| far below s is nearest to 0 by a wide margin. */
int orc_e2m1_code(float y, double s)
{
    int sign = signbit(y) ? 8 : 0;
    double a = fabs((double)y);
    if (s == 0.0) return sign;
    if (a >= 6.0 * s) return sign | 7;
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(a - orc_e2m1_value(c) * s);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = c;
        }
    }
    return sign | best;
}

/* ------------------------------------------------------------------------ */
/* RoPE table.  Release post, section "YaRN context extension": theta 1e7,
 * a quarter of the dims rotary, context extended by linear scaling of the
 * position.  For pair i < R/2 (R = rotary_dim):
 *   inv_i = theta^(-(2 i)/R),  angle = (pos / pos_scale) * inv_i,
 * evaluated in double with libm, then rounded once to float.
 * cos_out/sin_out are [max_pos][R/2]. */
void orc_rope_table(double theta, int rotary_dim, double pos_scale, int max_pos,
                    float* cos_out, float* sin_out)
{
    int half = rotary_dim / 2;
    for (int p = 0; p < max_pos; ++p) {
        for (int i = 0; i < half; ++i) {
            double inv = pow(theta, -(2.0 * i) / (double)rotary_dim);
            double ang = ((double)p / pos_scale) * inv;
            cos_out[(size_t)p * half + i] = (float)cos(ang);
            sin_out[(size_t)p * half + i] = (float)sin(ang);
        }
    }
}

/* Rotate-half RoPE on the first R dims of a float row (pairs i, i + R/2),
 * binary32, each product and sum rounded on its own:
 *   x'[i]       = (x[i] c_i) - (x[i+R/2] s_i)
 *   x'[i+R/2]   = (x[i+R/2] c_i) + (x[i] s_i)
 * Dims R..127 are unchanged. */
void orc_rope_apply(float* x, int rotary_dim, const float* c, const float* s)
{
    int half = rotary_dim / 2;
    for (int i = 0; i < half; ++i) {
        float a = x[i], b = x[i + half];
        float ac = a * c[i], bs = b * s[i];
        float bc = b * c[i], as = a * s[i];
        x[i] = ac - bs;
        x[i + half] = bc + as;
    }
}

/* Hadamard rotation of a 128-vector (release post, NVFP4 section, bullet 2):
 * y = H x / sqrt(128), H the Sylvester (Walsh) matrix H[i][j] =
 * (-1)^popcount(i & j).  Computed with the fast Walsh-Hadamard transform in
 * binary32: for h = 1, 2, 4, ..., 64 and each pair (j, j+h) with bit h of j
 * clear, (a, b) -> (a + b, a - b); then every entry is multiplied by the
 * float nearest 2^-3.5 = 1/sqrt(128). */
void orc_hadamard128(float* x)
{
    for (int h = 1; h < ORC_D; h <<= 1) {
        for (int j = 0; j < ORC_D; ++j) {
            if (j & h) continue;
            float a = x[j], b = x[j + h];
            x[j] = a + b;
            x[j + h] = a - b;
        }
    }
    const float inv_sqrt128 = (float)0.08838834764831845; /* 2^-3.5 */
    for (int j = 0; j < ORC_D; ++j) x[j] = x[j] * inv_sqrt128;
}

/* Quantize one 128-element row to NVFP4 (release post, NVFP4 section):
 *   1. RoPE on the first rotary_dim dims (K and Q only; pass rotary_dim 0
 *      for V or when the row carries no position);
 *   2. Hadamard rotation when `hadamard` is non-zero (K and Q only).  With
 *      hadamard == 2 (a variant, not the post's: a randomized rotation) the
 *      elements whose bit is set in the 128-bit mask `signs` (bit j of
 *      element j: word j / 32, bit j % 32) are negated first, so the row is
 *      multiplied by H D / sqrt(128) with D = diag(+-1); Q and K get the same
 *      D, and (H D q) . (H D k) = q . k still holds;
 *   3. per block of 16: amax, E4M3 scale nearest amax/6;
 *   4. per element: E2M1 code against the block scale;
 *   5. pack two codes per byte, element 2j in the low nibble of byte j.
 * codes: 64 bytes, scales: 8 bytes (block b = elements 16b..16b+15). */
void orc_quant_row(const float* x_in, int rotary_dim, const float* c, const float* s,
                   int hadamard, const uint32_t* signs, uint8_t* codes, uint8_t* scales)
{
    float x[ORC_D];
    memcpy(x, x_in, sizeof x);
    if (rotary_dim > 0) orc_rope_apply(x, rotary_dim, c, s);
    if (hadamard == 2)
        for (int j = 0; j < ORC_D; ++j)
            if ((signs[j >> 5] >> (j & 31)) & 1u) x[j] = -x[j];
    if (hadamard) orc_hadamard128(x);
    int nib[ORC_D];
    for (int b = 0; b < ORC_NBLK; ++b) {
        float amax = 0.0f;
        for (int i = 0; i < ORC_BLOCK; ++i) {
            float a = fabsf(x[b * ORC_BLOCK + i]);
            if (a > amax) amax = a;
        }
        int sc = orc_e4m3_scale_code(amax);
        scales[b] = (uint8_t)sc;
        double sv = orc_e4m3_value(sc);
        for (int i = 0; i < ORC_BLOCK; ++i)
            nib[b * ORC_BLOCK + i] = orc_e2m1_code(x[b * ORC_BLOCK + i], sv);
    }
    for (int j = 0; j < ORC_ROW_CODE; ++j)
        codes[j] = (uint8_t)(nib[2 * j] | (nib[2 * j + 1] << 4));
}

/* Dequantize a row: element = e2m1(code) * e4m3(scale), exact in double. */
void orc_dequant_row(const uint8_t* codes, const uint8_t* scales, double* out)
{
    for (int d = 0; d < ORC_D; ++d) {
        int byte = codes[d / 2];
        int nibble = (d & 1) ? (byte >> 4) : (byte & 15);
        out[d] = orc_e2m1_value(nibble) * orc_e4m3_value(scales[d / ORC_BLOCK]);
    }
}

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16 (fp16): the V storage of the variant the release post
 * names as upstream's ("fp16 V storage", NVFP4 section, bullet 2).  1 sign,
 * 5 exponent bits (bias 15), 10 mantissa bits; subnormals are multiples of
 * 2^-24; largest finite 65504. */

/* binary16 bits of the float x, rounded to nearest with ties to even (the
 * IEEE default), overflowing to infinity, NaN kept a (quiet) NaN.  Written
 * from the definition: |x| is split into its binary exponent E and the
 * integer count of binary16 ulps 2^(E-10) (2^-24 below 2^-14), which is
 * rounded with rint (ties to even under the default rounding mode); every
 * step before the rounding is exact in double.  Infinities stay infinite. */
uint16_t orc_f32_to_f16(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x)) return sign | 0x7E00;
    if (isinf(a)) return sign | 0x7C00;
    if (a < ldexp(1.0, -14)) {                         /* subnormal or zero */
        double m = rint(a * 16777216.0);                /* units of 2^-24; 1024 = 2^-14 */
        return sign | (uint16_t)m;
    }
    int e;
    frexp(a, &e);                                       /* a = f 2^e, f in [0.5, 1) */
    int E = e - 1;                                      /* a in [2^E, 2^(E+1)) */
    double m = rint(ldexp(a, 10 - E));                  /* [1024, 2048] */
    if (m == 2048.0) {
        m = 1024.0;
        E += 1;
    }
    if (E > 15) return sign | 0x7C00;                   /* infinity */
    return sign | (uint16_t)(((E + 15) << 10) | ((int)m - 1024));
}

/* The value of binary16 bits h, exactly, in double. */
double orc_f16_value(uint16_t h)
{
    int e = (h >> 10) & 31, m = h & 1023;
    double mag;
    if (e == 31) mag = m ? NAN : INFINITY;
    else if (e == 0) mag = ldexp((double)m, -24);
    else mag = ldexp(1024.0 + m, e - 25);
    return (h & 0x8000) ? -mag : mag;
}

void orc_f32_to_f16_array(const float* x, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(x[i]);
}

/* ------------------------------------------------------------------------ */
/* Paged pool.  One block per (layer, page, kv-head), blocks in
 * [layer][page][kv_head] order; a slot is page*64 + t.
 *
 * v_format 0 (NVFP4 V, the release post's format): 9216 bytes per block.
 * Inside a block (64 tokens t, code byte j):
 *   K codes    at        (t/16)*1024 + (j/16)*256 + (t%16)*16 + (j%16)
 *   V codes    at 4096 + (t/4)*256  + (j/4)*16   + (t%4)*4   + (j%4)
 *   K scales   at 8192 + t*8 + b        (row-major, release post bullet 4)
 *   V scales   at 8704 + t*8 + b
 * Per token and kv-head: 2 * (64 + 8) = 144 bytes.
 *
 * v_format 1 (fp16 V, NVFP4 K; the upstream storage named in bullet 2):
 * 20992 bytes per block, 328 per token and kv-head.
 *   K codes    as above
 *   V (fp16)   element d of token t at 4096 + (t/32)*8192 + (d%8)*1024
 *              + (((t%16)/4)*16 + d/8)*16 + ((t%4) + 4*((t%32)/16))*2,
 *              2 bytes little-endian
 *   K scales   at 20480 + t*8 + b
 * (The V order puts the eight fp16 values one lane of a 16x16x32 matrix
 * instruction reads next to each other; it is this library's choice, the
 * pages give none.) */
static size_t orc_block_bytes(int v_format) { return v_format ? 20992 : 9216; }
static int orc_kscale_off(int v_format) { return v_format ? 20480 : 8192; }

size_t orc_pool_bytes(int num_layers, int64_t num_pages, int num_kv_heads, int v_format)
{
    return (size_t)num_layers * (size_t)num_pages * (size_t)num_kv_heads * orc_block_bytes(v_format);
}

static size_t orc_block_base(int64_t num_pages, int hkv, int layer, int64_t page, int kvh, int v_format)
{
    return (((size_t)layer * (size_t)num_pages + (size_t)page) * (size_t)hkv + (size_t)kvh)
           * orc_block_bytes(v_format);
}

static size_t orc_kcode_off(int t, int j) { return (size_t)((t / 16) * 1024 + (j / 16) * 256 + (t % 16) * 16 + (j % 16)); }
static size_t orc_vcode_off(int t, int j) { return (size_t)(4096 + (t / 4) * 256 + (j / 4) * 16 + (t % 4) * 4 + (j % 4)); }
static size_t orc_v16_off(int t, int d)
{
    return (size_t)(4096 + (t / 32) * 8192 + (d % 8) * 1024 + (((t % 16) / 4) * 16 + d / 8) * 16
                    + ((t % 4) + 4 * ((t % 32) / 16)) * 2);
}

/* Read the codes and scales of one cached NVFP4 row.  which = 0 for K, 1 for
 * V (v_format 0 only). */
void orc_pool_read_row(const uint8_t* pool, int64_t num_pages, int hkv, int layer,
                       int64_t slot, int kvh, int which, int v_format, uint8_t* codes, uint8_t* scales)
{
    int64_t page = slot / ORC_PAGE;
    int t = (int)(slot % ORC_PAGE);
    const uint8_t* blk = pool + orc_block_base(num_pages, hkv, layer, page, kvh, v_format);
    for (int j = 0; j < ORC_ROW_CODE; ++j)
        codes[j] = blk[which ? orc_vcode_off(t, j) : orc_kcode_off(t, j)];
    for (int b = 0; b < ORC_NBLK; ++b)
        scales[b] = blk[(which ? 8704 : orc_kscale_off(v_format)) + t * 8 + b];
}

/* Read the 128 fp16 V values (bits) of one cached row of a v_format 1 pool. */
void orc_pool_read_v16(const uint8_t* pool, int64_t num_pages, int hkv, int layer, int64_t slot, int kvh,
                       uint16_t* out)
{
    int64_t page = slot / ORC_PAGE;
    int t = (int)(slot % ORC_PAGE);
    const uint8_t* blk = pool + orc_block_base(num_pages, hkv, layer, page, kvh, 1);
    for (int d = 0; d < ORC_D; ++d) {
        size_t o = orc_v16_off(t, d);
        out[d] = (uint16_t)(blk[o] | (blk[o + 1] << 8));
    }
}

static void orc_pool_write_row(uint8_t* pool, int64_t num_pages, int hkv, int layer,
                               int64_t slot, int kvh, int which, int v_format,
                               const uint8_t* codes, const uint8_t* scales)
{
    int64_t page = slot / ORC_PAGE;
    int t = (int)(slot % ORC_PAGE);
    uint8_t* blk = pool + orc_block_base(num_pages, hkv, layer, page, kvh, v_format);
    for (int j = 0; j < ORC_ROW_CODE; ++j)
        blk[which ? orc_vcode_off(t, j) : orc_kcode_off(t, j)] = codes[j];
    for (int b = 0; b < ORC_NBLK; ++b)
        blk[(which ? 8704 : orc_kscale_off(v_format)) + t * 8 + b] = scales[b];
}

static void orc_pool_write_v16(uint8_t* pool, int64_t num_pages, int hkv, int layer, int64_t slot, int kvh,
                               const float* v)
{
    int64_t page = slot / ORC_PAGE;
    int t = (int)(slot % ORC_PAGE);
    uint8_t* blk = pool + orc_block_base(num_pages, hkv, layer, page, kvh, 1);
    for (int d = 0; d < ORC_D; ++d) {
        uint16_t h = orc_f32_to_f16(v[d]);
        size_t o = orc_v16_off(t, d);
        blk[o] = (uint8_t)(h & 0xFF);
        blk[o + 1] = (uint8_t)(h >> 8);
    }
}

/* Append n_tok tokens (release post, NVFP4 section, bullet 3): for every
 * token and kv-head, K gets RoPE (at positions[i]) + Hadamard + NVFP4, V gets
 * NVFP4 only (v_format 0) or is rounded to fp16 (v_format 1), and both rows
 * are written into the slot's page.
 * k, v: [n_tok][hkv][128] floats (bf16 inputs are widened exactly first).
 * cos_tab/sin_tab: [max_pos][rotary_dim/2]. */
void orc_append(uint8_t* pool, int64_t num_pages, int hkv, int rotary_dim, int hadamard,
                const uint32_t* signs, int layer, int n_tok, const float* k, const float* v,
                const int64_t* slots, const int32_t* positions,
                const float* cos_tab, const float* sin_tab, int v_format)
{
    int half = rotary_dim / 2;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < n_tok; ++i) {
        for (int g = 0; g < hkv; ++g) {
            uint8_t codes[ORC_ROW_CODE], scales[ORC_NBLK];
            const float* c = rotary_dim > 0 ? cos_tab + (size_t)positions[i] * half : NULL;
            const float* s = rotary_dim > 0 ? sin_tab + (size_t)positions[i] * half : NULL;
            orc_quant_row(k + ((size_t)i * hkv + g) * ORC_D, rotary_dim, c, s, hadamard, signs,
                          codes, scales);
            orc_pool_write_row(pool, num_pages, hkv, layer, slots[i], g, 0, v_format, codes, scales);
            if (v_format) {
                orc_pool_write_v16(pool, num_pages, hkv, layer, slots[i], g, v + ((size_t)i * hkv + g) * ORC_D);
            } else {
                orc_quant_row(v + ((size_t)i * hkv + g) * ORC_D, 0, NULL, NULL, 0, NULL, codes, scales);
                orc_pool_write_row(pool, num_pages, hkv, layer, slots[i], g, 1, 0, codes, scales);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Decode attention over the pool (release post, NVFP4 section, bullets 1-3).
 * For sequence n and query head h (kv head g = h / (hq/hkv)):
 *   Qhat  = dequant(quant(q[n][h]))  with RoPE at q_pos[n] and the Hadamard
 *           rotation (the same row quantizer as K);
 *   z_t   = sm_scale * sum_d Qhat[d] * Khat_t[d],  t = 0 .. seq_lens[n]-1,
 *           Khat/Vhat dequantized from the slots page_table[n][t/64]*64 + t%64;
 *   o     = sum_t softmax(z)_t * Vhat_t.
 * All of it in double.  q: [n_seq][hq][128] floats; out: [n_seq][hq][128].
 * With v_rows (one sequence only) the V values are taken from v_rows
 * [T][hkv][128] instead of the pool: the K-only-quantized variant of a
 * quality study (V kept in a 16-bit format by the caller).  v_format 1: the
 * pool keeps V in fp16 (the values are read from it exactly). */
void orc_decode_attention(const uint8_t* pool, int64_t num_pages, int hkv, int layer,
                          int rotary_dim, int hadamard, const uint32_t* signs, int n_seq, int hq,
                          const float* q, const int32_t* q_pos,
                          const float* cos_tab, const float* sin_tab,
                          const int32_t* page_table, int page_table_stride,
                          const int32_t* seq_lens, double sm_scale, const float* v_rows,
                          int v_format, double* out)
{
    int grp = hq / hkv, half = rotary_dim / 2;
    for (int n = 0; n < n_seq; ++n) {
        int T = seq_lens[n];
        for (int g = 0; g < hkv; ++g) {
            double* qh = malloc(sizeof(double) * (size_t)grp * ORC_D);
            double* z = malloc(sizeof(double) * (size_t)grp * (size_t)T);
            for (int r = 0; r < grp; ++r) {
                uint8_t codes[ORC_ROW_CODE], scales[ORC_NBLK];
                const float* c = rotary_dim > 0 ? cos_tab + (size_t)q_pos[n] * half : NULL;
                const float* s = rotary_dim > 0 ? sin_tab + (size_t)q_pos[n] * half : NULL;
                orc_quant_row(q + ((size_t)n * hq + g * grp + r) * ORC_D, rotary_dim, c, s,
                              hadamard, signs, codes, scales);
                orc_dequant_row(codes, scales, qh + (size_t)r * ORC_D);
            }
            /* scores */
#pragma omp parallel for schedule(static)
            for (int t = 0; t < T; ++t) {
                uint8_t codes[ORC_ROW_CODE], scales[ORC_NBLK];
                double kh[ORC_D];
                int64_t slot = (int64_t)page_table[(size_t)n * page_table_stride + t / ORC_PAGE]
                               * ORC_PAGE + t % ORC_PAGE;
                orc_pool_read_row(pool, num_pages, hkv, layer, slot, g, 0, v_format, codes, scales);
                orc_dequant_row(codes, scales, kh);
                for (int r = 0; r < grp; ++r) {
                    double acc = 0.0;
                    for (int d = 0; d < ORC_D; ++d) acc += qh[(size_t)r * ORC_D + d] * kh[d];
                    z[(size_t)r * T + t] = sm_scale * acc;
                }
            }
            /* softmax weights and weighted sum of V, per query head */
            for (int r = 0; r < grp; ++r) {
                double mx = -INFINITY;
                for (int t = 0; t < T; ++t) if (z[(size_t)r * T + t] > mx) mx = z[(size_t)r * T + t];
                for (int t = 0; t < T; ++t) z[(size_t)r * T + t] = exp(z[(size_t)r * T + t] - mx);
            }
            double* o = out + ((size_t)n * hq + g * grp) * ORC_D;
            /* Weighted sum of V over fixed chunks of tokens, the chunks added
             * in token order, so the result does not depend on the thread
             * count. */
            const int CH = 4096;
            int nch = (T + CH - 1) / CH;
            double* part = calloc((size_t)nch * grp * (ORC_D + 1), sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
            for (int ch = 0; ch < nch; ++ch) {
                double* acc = part + (size_t)ch * grp * (ORC_D + 1);
                int t1 = (ch + 1) * CH < T ? (ch + 1) * CH : T;
                for (int t = ch * CH; t < t1; ++t) {
                    uint8_t codes[ORC_ROW_CODE], scales[ORC_NBLK];
                    double vh[ORC_D];
                    int64_t slot = (int64_t)page_table[(size_t)n * page_table_stride + t / ORC_PAGE]
                                   * ORC_PAGE + t % ORC_PAGE;
                    if (v_rows != NULL) {
                        for (int d = 0; d < ORC_D; ++d) vh[d] = v_rows[((size_t)t * hkv + g) * ORC_D + d];
                    } else if (v_format) {
                        uint16_t h16[ORC_D];
                        orc_pool_read_v16(pool, num_pages, hkv, layer, slot, g, h16);
                        for (int d = 0; d < ORC_D; ++d) vh[d] = orc_f16_value(h16[d]);
                    } else {
                        orc_pool_read_row(pool, num_pages, hkv, layer, slot, g, 1, 0, codes, scales);
                        orc_dequant_row(codes, scales, vh);
                    }
                    for (int r = 0; r < grp; ++r) {
                        double p = z[(size_t)r * T + t];
                        acc[(size_t)r * (ORC_D + 1) + ORC_D] += p;
                        for (int d = 0; d < ORC_D; ++d) acc[(size_t)r * (ORC_D + 1) + d] += p * vh[d];
                    }
                }
            }
            double* lsum = calloc((size_t)grp, sizeof(double));
            memset(o, 0, sizeof(double) * (size_t)grp * ORC_D);
            for (int ch = 0; ch < nch; ++ch)
                for (int r = 0; r < grp; ++r) {
                    const double* acc = part + ((size_t)ch * grp + r) * (ORC_D + 1);
                    for (int d = 0; d < ORC_D; ++d) o[(size_t)r * ORC_D + d] += acc[d];
                    lsum[r] += acc[ORC_D];
                }
            free(part);
            for (int r = 0; r < grp; ++r)
                for (int d = 0; d < ORC_D; ++d) o[(size_t)r * ORC_D + d] /= lsum[r];
            free(lsum);
            free(z);
            free(qh);
        }
    }
}

/* Unquantized reference (reported, not gated): the same attention on the
 * raw q, k, v rows with RoPE applied in binary32 as above, no Hadamard (it
 * cancels in q.k), no quantization; double precision throughout.
 * k, v: [T][hkv][128] for one sequence in token order; q: [hq][128]. */
void orc_reference_attention(int hkv, int hq, int T, int rotary_dim,
                             const float* q, int32_t q_pos, const float* k, const float* v,
                             const int32_t* k_pos, const float* cos_tab, const float* sin_tab,
                             double sm_scale, double* out)
{
    int grp = hq / hkv, half = rotary_dim / 2;
    double* z = malloc(sizeof(double) * (size_t)T);
    for (int h = 0; h < hq; ++h) {
        int g = h / grp;
        float qr[ORC_D];
        memcpy(qr, q + (size_t)h * ORC_D, sizeof qr);
        if (rotary_dim > 0)
            orc_rope_apply(qr, rotary_dim, cos_tab + (size_t)q_pos * half, sin_tab + (size_t)q_pos * half);
        double mx = -INFINITY;
#pragma omp parallel for schedule(static) reduction(max : mx)
        for (int t = 0; t < T; ++t) {
            float kr[ORC_D];
            memcpy(kr, k + ((size_t)t * hkv + g) * ORC_D, sizeof kr);
            if (rotary_dim > 0)
                orc_rope_apply(kr, rotary_dim, cos_tab + (size_t)k_pos[t] * half,
                               sin_tab + (size_t)k_pos[t] * half);
            double acc = 0.0;
            for (int d = 0; d < ORC_D; ++d) acc += (double)qr[d] * (double)kr[d];
            z[t] = sm_scale * acc;
            if (z[t] > mx) mx = z[t];
        }
        double l = 0.0;
        double* o = out + (size_t)h * ORC_D;
        for (int d = 0; d < ORC_D; ++d) o[d] = 0.0;
        for (int t = 0; t < T; ++t) {
            double p = exp(z[t] - mx);
            l += p;
            const float* vr = v + ((size_t)t * hkv + g) * ORC_D;
            for (int d = 0; d < ORC_D; ++d) o[d] += p * (double)vr[d];
        }
        for (int d = 0; d < ORC_D; ++d) o[d] /= l;
    }
    free(z);
}
