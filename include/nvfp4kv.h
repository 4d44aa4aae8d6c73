/*
 * nvfp4kv.h -- attention over a 4-bit NVFP4 KV cache on AMD Instinct MI355X
 * (gfx950).  C ABI of libnvfp4kv.so.
 *
 * The method is the one described in the release post of the gzenz/ninfer
 * fork (prismix.dev, news item 833001997676), section "NVFP4 KV cache (from
 * scratch)":
 *   - K and V are stored as NVFP4: 4-bit E2M1 elements, one E4M3 scale per
 *     16 elements, scales kept row-major without swizzle (bullets 1 and 4);
 *   - K and Q are rotated by a 128-point Hadamard transform before they are
 *     quantized, V is not rotated (bullet 2);
 *   - Q is quantized to NVFP4 as well; V is dequantized for the PV product
 *     (bullet 1);
 *   - the current token's K and V are quantized in place during decode,
 *     without a separate quantization pass (bullet 3);
 *   - 144 bytes per token per KV head (the "Result" line).
 * RoPE follows section "YaRN context extension" of the same post: rotary on a
 * leading part of the head (a quarter of it in the post's model), theta 1e7,
 * longer contexts by linear scaling of the position.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless a comment says "host".  The caller
 *     owns every buffer (pool, inputs, outputs, workspace) and keeps it alive
 *     until the work queued on `stream` has finished.  The library never
 *     allocates or frees device memory, never synchronizes, and keeps no
 *     device state.
 *   - All work is queued on `stream` in call order.  Append a token before
 *     the decode that must see it, on the same stream.
 *   - Arguments are checked on the host before anything is queued.  A bad
 *     argument returns a negative nvfp4kv_status and leaves a message for
 *     nvfp4kv_last_error(); nothing is queued then.  Device-side contents
 *     (slots, page ids, positions, sequence lengths) are trusted: values
 *     outside the documented ranges give undefined results.
 *   - No C++ exception crosses this interface.
 */
#ifndef NVFP4KV_H
#define NVFP4KV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4KV_OK = 0,
    NVFP4KV_ERR_INVALID_ARG = -1, /* null pointer, size or index out of range */
    NVFP4KV_ERR_UNSUPPORTED = -2, /* head_dim != 128, page_size != 64, ... */
    NVFP4KV_ERR_WORKSPACE = -3,   /* workspace too small or misaligned */
    NVFP4KV_ERR_HIP = -4          /* the HIP runtime reported an error */
} nvfp4kv_status;

typedef enum { NVFP4KV_F32 = 0, NVFP4KV_BF16 = 1 } nvfp4kv_dtype;

/* Byte layout of the pool (device memory, caller-owned, 256-byte aligned).
 * One block per (layer, page, kv head), blocks ordered [layer][page][kv_head].
 * A slot is page * 64 + t with t the token's place in its page.  Code byte j
 * of a row holds elements 2j (low nibble) and 2j+1 (high nibble).
 * v_format 0 (NVFP4 K and V, the release post's format): 9216 bytes a block,
 *   [   0, 4096) K codes, byte j of token t at (t/16)*1024 + (j/16)*256 + (t%16)*16 + j%16
 *   [4096, 8192) V codes, byte j of token t at 4096 + (t/4)*256 + (j/4)*16 + (t%4)*4 + j%4
 *   [8192, 8704) K scales, row-major: scale of block b (elements 16b..16b+15) of token t at 8192 + 8t + b
 *   [8704, 9216) V scales, row-major: at 8704 + 8t + b
 * v_format 1 (NVFP4 K, V in IEEE fp16: the upstream storage the release
 * post compares against, NVFP4 section, bullet 2): 20992 bytes a block,
 *   [    0,  4096) K codes as above
 *   [ 4096, 20480) V, element d of token t (fp16, little-endian) at
 *                  4096 + (t/32)*8192 + (d%8)*1024 + (((t%16)/4)*16 + d/8)*16 + ((t%4) + 4*((t%32)/16))*2
 *   [20480, 20992) K scales, row-major: at 20480 + 8t + b
 * The code and fp16 tilings put the 16 bytes that one lane of a 16x16x32
 * matrix instruction needs next to each other; the scales stay row-major as
 * the release post specifies.  K rows are stored rotated (Hadamard domain). */
typedef struct {
    void* base;             /* device pointer to the pool */
    int64_t num_pages;      /* pages per layer; page ids index [0, num_pages) */
    int32_t num_layers;     /* >= 1 */
    int32_t num_kv_heads;   /* >= 1 */
    int32_t head_dim;       /* must be 128 */
    int32_t page_size;      /* must be 64 */
    int32_t rotary_dim;     /* RoPE dims at the head's start: 0..128, even (pairs
                               i, i + rotary_dim/2); a multiple of 16 takes
                               the faster rotation, other even widths are
                               exact too */
    int32_t hadamard;       /* 1: rotate K and Q before quantizing; 0: do not;
                               2: rotate after negating the elements marked in
                               hadamard_signs (a randomized rotation, a variant
                               the release post does not use) */
    uint32_t hadamard_signs[4]; /* hadamard 2 only: element j of K and Q rows is
                                   negated before the transform when bit j % 32
                                   of word j / 32 is set; the caller draws it */
    float k_scale;          /* per-tensor global scale of K, 0 meaning 1: append
                               multiplies each K input element by the binary32
                               1/k_scale before RoPE and quantization, so the
                               E4M3 block scales see amax/k_scale; dequant and
                               decode multiply the stored values back by it.
                               0 or a finite value in [2^-64, 2^64].  NVFP4's
                               second scaling level (a tensor-wide FP32 factor
                               over the block scales); the release post keeps
                               it at 1 */
    float v_scale;          /* the same for V */
    int32_t v_format;       /* 0: V in NVFP4 (144 bytes per token per kv head);
                               1: V in fp16 (328 bytes; each element times the
                               binary32 1/v_scale, rounded to nearest even).
                               The fp16 form is a comparison variant: decode
                               takes it for up to 8 query heads per kv head
                               and one query token (nvfp4kv_decode_attn,
                               _static, _splits); multi-token decode and the
                               read probe refuse it (NVFP4KV_ERR_UNSUPPORTED) */
} nvfp4kv_pool;

/* Bytes the pool needs: num_layers * num_pages * num_kv_heads * 64 * 144,
 * i.e. 144 bytes per token per kv head (release post, NVFP4 section, the
 * "Result" line: 2 x (64 code bytes + 8 E4M3 scale bytes) for a 128-element
 * head); 328 instead of 144 with v_format 1 (64 + 8 for K, 256 for fp16 V).
 * Host only.  Returns 0 if `p` is null or its sizes are invalid. */
size_t nvfp4kv_pool_bytes(const nvfp4kv_pool* p);

/* RoPE table on the HOST (section "YaRN context extension"): for position
 * pos < max_pos and pair i < rotary_dim/2,
 *   angle = (pos / pos_scale) * theta^(-(2 i)/rotary_dim)
 * evaluated in double, cos and sin rounded once to float, written to host
 * arrays cos_out/sin_out laid out [max_pos][rotary_dim/2].  pos_scale is the
 * linear position-scaling factor (1 = none).  Copy the table to the device
 * and pass it to nvfp4kv_append and nvfp4kv_decode_attn. */
int nvfp4kv_rope_table(double theta, int32_t rotary_dim, double pos_scale, int32_t max_pos,
                       float* cos_out, float* sin_out);

/* Append n_tok tokens to one layer of the pool (bullets 1-4 of the NVFP4
 * section): K rows get RoPE at positions[i], then the Hadamard rotation if
 * the pool's `hadamard` is 1; V rows get neither.  Each row is quantized to
 * NVFP4 (E4M3 scale nearest amax/6 per 16 elements, E2M1 codes rounded to
 * nearest even) and written to slot slots[i], overwriting what was there.
 *   k, v       [n_tok][num_kv_heads][128], dtype in_dtype (bf16 or f32)
 *   slots      [n_tok] int64, page * 64 + offset, page < num_pages
 *   positions  [n_tok] int32, < max_pos (read only when rotary_dim > 0)
 *   rope_cos/rope_sin [max_pos][rotary_dim/2] float, 16-byte aligned (may
 *              be null when rotary_dim == 0; nvfp4kv_rope_table fills them)
 * Two tokens with the same slot in one call race. */
int nvfp4kv_append(const nvfp4kv_pool* p, int32_t layer, int32_t n_tok,
                   const void* k, const void* v, nvfp4kv_dtype in_dtype,
                   const int64_t* slots, const int32_t* positions,
                   const float* rope_cos, const float* rope_sin, int32_t max_pos,
                   hipStream_t stream);

/* Workspace bytes nvfp4kv_decode_attn needs for this shape: the split
 * partials of the decode attention of the NVFP4 section's bullets 1-3 (the
 * release post does not describe how its decode kernel splits the work; the
 * split and its partials are this library's).  Host only; the caller
 * allocates the workspace.  pages_per_split 0 selects the library's own
 * split plan; the same value must be passed to nvfp4kv_decode_attn.
 * Returns 0 on invalid arguments (the reason is left for
 * nvfp4kv_last_error). */
size_t nvfp4kv_decode_workspace_bytes(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_q_heads,
                                      int64_t max_seq_len, int32_t pages_per_split);

/* One decode step of attention for n_seq sequences (bullets 1-3 of the NVFP4
 * section).  For sequence n and query head h (kv head h / (n_q_heads /
 * num_kv_heads)): the query gets RoPE at q_positions[n] and the Hadamard
 * rotation (when the pool has it), is quantized to NVFP4 and dequantized;
 * scores against the dequantized cached K of tokens 0 .. seq_lens[n]-1 are
 * scaled by sm_scale, softmax-normalized, and weight the dequantized V.
 * Two kernels: the pages of all (sequence, kv head) pairs are split evenly
 * over the decode wavefronts, each writing partial results to the
 * workspace (and quantizing the current token and the queries it needs);
 * a reduce kernel combines them.
 *   q           [n_seq][n_q_heads][128], dtype q_dtype, before RoPE
 *   k_new/v_new [n_seq][num_kv_heads][128], dtype q_dtype, before RoPE: the
 *               current token's K and V, or both null.  When given, the
 *               decode kernel quantizes them into the cache slot of token
 *               seq_lens[n]-1 (RoPE at q_positions[n] and the rotation on K),
 *               bit for bit as nvfp4kv_append would, before that slot's page
 *               is read: the step needs no separate append.  Only that slot
 *               is written.
 *   q_positions [n_seq] int32
 *   page_table  [n_seq][page_table_stride] int32 page ids; token t of
 *               sequence n sits in slot page_table[n][t/64]*64 + t%64
 *   seq_lens    [n_seq] int32, 1 <= seq_lens[n] <= max_seq_len, counting the
 *               token appended in this step
 *   max_seq_len host value, sizes the grid
 *   sm_scale    >= 0 (1/sqrt(128) for plain attention)
 *   out         [n_seq][n_q_heads][128] float
 *   workspace   at least nvfp4kv_decode_workspace_bytes(...) bytes, 256-byte
 *               aligned; its contents on entry do not matter
 *   pages_per_split 0 = automatic, else 1..4096
 * n_q_heads / num_kv_heads must be an integer from 1 to 16. */
int nvfp4kv_decode_attn(const nvfp4kv_pool* p, int32_t layer, int32_t n_seq, int32_t n_q_heads,
                        const void* q, const void* k_new, const void* v_new,
                        nvfp4kv_dtype q_dtype, const int32_t* q_positions,
                        const float* rope_cos, const float* rope_sin, int32_t max_pos,
                        const int32_t* page_table, int32_t page_table_stride,
                        const int32_t* seq_lens, int64_t max_seq_len, float sm_scale,
                        float* out, void* workspace, size_t workspace_bytes,
                        int32_t pages_per_split, hipStream_t stream);

/* nvfp4kv_decode_attn without a workspace argument and without allocating
 * anything: for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The split partials go to the library's own workspace, a device array of
 * NVFP4KV_STATIC_WORKSPACE_BYTES that every GPU the library runs on holds
 * until the process ends.  Arguments, outputs and results are those of
 * nvfp4kv_decode_attn with the same pages_per_split.  A call whose workspace
 * (nvfp4kv_decode_workspace_bytes) would exceed the array returns
 * NVFP4KV_ERR_WORKSPACE before anything is queued.  The array keeps the last
 * call's contents (nothing in it needs clearing); calls that overlap on one
 * GPU (queued on different streams without ordering) race on it. */
#define NVFP4KV_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)
int nvfp4kv_decode_attn_static(const nvfp4kv_pool* p, int32_t layer, int32_t n_seq, int32_t n_q_heads,
                               const void* q, const void* k_new, const void* v_new,
                               nvfp4kv_dtype q_dtype, const int32_t* q_positions,
                               const float* rope_cos, const float* rope_sin, int32_t max_pos,
                               const int32_t* page_table, int32_t page_table_stride,
                               const int32_t* seq_lens, int64_t max_seq_len, float sm_scale, float* out,
                               int32_t pages_per_split, hipStream_t stream);

/* The two stages of nvfp4kv_decode_attn, for callers that combine split
 * partials themselves (for example across devices) or time the stages apart.
 * nvfp4kv_decode_attn_splits takes the arguments of nvfp4kv_decode_attn
 * except `out` and writes only the workspace.  Work layout: the pages of
 * segment g = seq * num_kv_heads + kvh, segments in order, each segment
 * followed by 5 units of no work, form one flat list of TU units; the plan's
 * W ranges [w*TU/W, (w+1)*TU/W) split it, and every (segment, range) pair
 * whose pages overlap yields one partial in slot g + w.  Per query head h of
 * the group a partial holds:
 *   m       a reference in log2 units: scores enter as
 *           s = sm_scale * k_scale * log2(e) * (Q-hat . K-hat), with K-hat
 *           the stored (block-scaled) K values, so K's global scale is
 *           inside m;
 *   l       the weight sum, sum_t 2^(s_t - m + 8) over the pair's tokens;
 *   acc     sum_t 2^(s_t - m + 8) V-hat_t with V-hat the STORED V values,
 *           i.e. V / v_scale (V's global scale is not applied here).
 * Layout, each part starting at a 256-byte boundary: acc at float offset
 * (slot * group + h) * 128 for slots 0 .. n_seq*num_kv_heads + W - 1; the
 * pairs (m, l) at float2 index slot * group + h.  Slots of pairs that do not
 * overlap are not written.
 * nvfp4kv_decode_reduce reads them and writes, per (sequence, query head),
 *   out = v_scale * sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
 * (M = max_s m_s; v_scale of the pool, 1 when unset): a caller combining
 * partials itself multiplies by v_scale too.  Both must get the same n_seq,
 * n_q_heads, max_seq_len and pages_per_split. */
int nvfp4kv_decode_attn_splits(const nvfp4kv_pool* p, int32_t layer, int32_t n_seq,
                               int32_t n_q_heads, const void* q, const void* k_new,
                               const void* v_new, nvfp4kv_dtype q_dtype,
                               const int32_t* q_positions, const float* rope_cos,
                               const float* rope_sin, int32_t max_pos, const int32_t* page_table,
                               int32_t page_table_stride, const int32_t* seq_lens,
                               int64_t max_seq_len, float sm_scale, void* workspace,
                               size_t workspace_bytes, int32_t pages_per_split, hipStream_t stream);

int nvfp4kv_decode_reduce(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_q_heads,
                          const int32_t* seq_lens, int64_t max_seq_len, float* out,
                          const void* workspace, size_t workspace_bytes, int32_t pages_per_split,
                          hipStream_t stream);

/* Decode attention for n_qtok new query tokens per sequence at once, causal
 * among them: the verification step of speculative decoding, where a draft
 * model proposes several tokens and the main model checks them in one step
 * (ai-manual.ru article on "Ninfer 4080", section "Key features": DFlash2
 * with K = 7 drafted tokens), or the tail of a chunked prefill.  The n_qtok
 * tokens are the last n_qtok of each sequence and must already be in the
 * cache (nvfp4kv_append).  Query token j of sequence n attends to the
 * sequence's tokens 0 .. seq_lens[n] - n_qtok + j; otherwise each query
 * token is treated as in nvfp4kv_decode_attn (RoPE at its own position,
 * Hadamard rotation, NVFP4 round trip).
 *   q           [n_seq][n_qtok][n_q_heads][128], dtype q_dtype, before RoPE
 *   q_positions [n_seq][n_qtok] int32 (read only when rotary_dim > 0)
 *   seq_lens    [n_seq] int32, n_qtok <= seq_lens[n] <= max_seq_len,
 *               counting the n_qtok tokens
 *   out         [n_seq][n_qtok][n_q_heads][128] float
 *   workspace   at least nvfp4kv_decode_multi_workspace_bytes(...) bytes,
 *               256-byte aligned; its contents on entry do not matter
 * Other arguments as in nvfp4kv_decode_attn.  The cache is read once per
 * floor(48 / (n_q_heads / num_kv_heads)) query tokens (a launch takes up to
 * 48 matrix columns, each a query head of one token), each such launch
 * followed by its reduce; 1 <= n_qtok <= 64.  n_qtok = 1 computes what
 * nvfp4kv_decode_attn computes without k_new/v_new.  The workspace is
 * reused by the launches in stream order. */
size_t nvfp4kv_decode_multi_workspace_bytes(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_qtok,
                                            int32_t n_q_heads, int64_t max_seq_len,
                                            int32_t pages_per_split);

int nvfp4kv_decode_attn_multi(const nvfp4kv_pool* p, int32_t layer, int32_t n_seq, int32_t n_qtok,
                              int32_t n_q_heads, const void* q, nvfp4kv_dtype q_dtype,
                              const int32_t* q_positions, const float* rope_cos,
                              const float* rope_sin, int32_t max_pos, const int32_t* page_table,
                              int32_t page_table_stride, const int32_t* seq_lens,
                              int64_t max_seq_len, float sm_scale, float* out, void* workspace,
                              size_t workspace_bytes, int32_t pages_per_split, hipStream_t stream);

/* Dequantize cached rows (release post, NVFP4 section, bullet 1: the V
 * operand of PV is the dequantized cache; element = E2M1 value * E4M3 block
 * scale, exact in f32 and bf16, times the pool's global scale).  K comes
 * back in the rotated domain (bullet 2) unless `unrotate` is 1, which applies
 * the Hadamard transform once more (it is its own inverse; the result then
 * carries float rounding).  A validation and export aid.
 *   slots       [n_tok] int64
 *   k_out/v_out [n_tok][num_kv_heads][128] of out_dtype; either may be null */
int nvfp4kv_dequant(const nvfp4kv_pool* p, int32_t layer, int32_t n_tok, const int64_t* slots,
                    void* k_out, void* v_out, nvfp4kv_dtype out_dtype, int32_t unrotate,
                    hipStream_t stream);

/* Bytes of one spilled page: every layer's and every kv head's block of one
 * page id, num_layers * num_kv_heads * (9216, or 20992 with v_format 1)
 * (host; 0 for an invalid pool). */
size_t nvfp4kv_page_bytes(const nvfp4kv_pool* p);

/* Host spill and restore of whole cache pages: the pinned host arena of the
 * release post's section "Multi-level prefix reuse with host-KV safety net"
 * (pages are copied device to host before eviction, and back on reuse).
 * nvfp4kv_spill_pages copies page page_ids[i] of every layer and kv head to
 * arena entry i; nvfp4kv_restore_pages copies arena entry i back into page
 * page_ids[i].  The bytes are copied unchanged, so a page can come back
 * under another page id (the page table then names the new id).
 *   page_ids    [n_pages] int32 in device memory or pinned host memory; ids
 *               outside [0, num_pages) are skipped (their arena entry is
 *               left as it was on spill)
 *   arena       [n_pages][num_layers][num_kv_heads][block bytes], at least
 *               n_pages * nvfp4kv_page_bytes(p) bytes, 16-byte aligned, in
 *               pinned host memory (hipHostMalloc) or in device memory of
 *               the current device; any other pointer is refused
 *               (NVFP4KV_ERR_INVALID_ARG) before anything is launched
 * One kernel, asynchronous on `stream`; the arena must stay allocated until
 * it has run.  The ids of a restore must be distinct: entries are copied in
 * parallel, so a page id listed twice ends with bytes of either entry, mixed
 * (a spill may list an id several times).  n_pages 0 does nothing. */
int nvfp4kv_spill_pages(const nvfp4kv_pool* p, int32_t n_pages, const int32_t* page_ids, void* arena,
                        size_t arena_bytes, hipStream_t stream);
int nvfp4kv_restore_pages(const nvfp4kv_pool* p, int32_t n_pages, const int32_t* page_ids,
                          const void* arena, size_t arena_bytes, hipStream_t stream);

/* Read-bandwidth probe of the decode access pattern (a measurement aid, not
 * a step of the method): reads every 9216-byte block of `layer` that
 * nvfp4kv_decode_attn over the same sequences reads (segment seq *
 * num_kv_heads + kvh holds pages 0 .. ceil(seq_lens[seq] / 64) - 1 of the
 * sequence, segments in order), split into n_waves equal ranges of that flat
 * list, one wavefront each, with the decode kernel's loads (nine 16-byte
 * non-temporal loads per lane and block, the next block in flight), and
 * writes the XOR of the 32-bit words wavefront w read to words[w].  The XOR
 * of all n_waves words is the XOR of every 32-bit word of those blocks,
 * whatever the split.
 *   page_table  [n_seq][page_table_stride] int32 page ids (device)
 *   seq_lens    [n_seq] int32 (device), >= 0
 *   words       [n_waves] uint32 (device)
 * Device-side contents are trusted, as for decode.  One kernel, asynchronous
 * on `stream`. */
int nvfp4kv_stream_read(const nvfp4kv_pool* p, int32_t layer, int32_t n_seq, const int32_t* page_table,
                        int32_t page_table_stride, const int32_t* seq_lens, int32_t n_waves, uint32_t* words,
                        hipStream_t stream);

/* Range checks of the device-side tables that the entry points above trust
 * (the header's conventions: slots, page ids, positions and sequence lengths
 * are not checked on the device), run on HOST copies of them.  A caller may
 * run them itself; the checked build of the library (libnvfp4kv_debug.so,
 * compiled with NVFP4KV_DEBUG=1) runs them inside every entry point on
 * copies it takes on the call's stream (which synchronizes that stream)
 * before anything is launched.  Each returns NVFP4KV_OK, or
 * NVFP4KV_ERR_INVALID_ARG with a message naming the first offending index
 * (nvfp4kv_last_error).  The release post's section "Also included" lists a
 * use-after-free that a missing stream synchronization caused: the checked
 * build is the tool for catching a bad table before a kernel reads with it.
 *   nvfp4kv_check_decode_tables: for each sequence n, n_qtok <= seq_lens[n]
 *       <= max_seq_len and page_table[n][j] in [0, num_pages) for the
 *       ceil(seq_lens[n] / 64) pages it uses; with rotary_dim > 0 and
 *       q_positions given, the n_seq * n_qtok positions in [0, max_pos)
 *   nvfp4kv_check_slots: slots in [0, num_pages * 64) and pairwise distinct
 *       (equal slots in one append race); with rotary_dim > 0 and positions
 *       given, positions in [0, max_pos)
 *   nvfp4kv_check_page_ids: with `distinct` (a restore), no page id inside
 *       the pool listed twice (ids outside the pool are skipped by contract)
 * nvfp4kv_checked_build returns 1 in the checked build, 0 otherwise. */
int nvfp4kv_check_decode_tables(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_qtok, const int32_t* page_table,
                                int32_t page_table_stride, const int32_t* seq_lens, int64_t max_seq_len,
                                const int32_t* q_positions, int32_t max_pos);
int nvfp4kv_check_slots(const nvfp4kv_pool* p, int32_t n_tok, const int64_t* slots, const int32_t* positions,
                        int32_t max_pos);
int nvfp4kv_check_page_ids(const nvfp4kv_pool* p, int32_t n_pages, const int32_t* page_ids, int32_t distinct);
int nvfp4kv_checked_build(void);

/* Message of the last failed call on this thread ("" if none).  Valid until
 * the next call on the same thread.  Not a step of the method: every entry
 * point reports failure as a status code and this message instead of
 * throwing (the release post's section "Also included" lists recovery from
 * allocation failures in its engine; here no exception ever crosses the C
 * interface). */
const char* nvfp4kv_last_error(void);

/* Library version string, e.g. "nvfp4kv 0.1.0 gfx950". */
const char* nvfp4kv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_H */
