// C ABI of libnvfp4kv: argument checks, split-K planning and kernel launches.
// Built with NVFP4KV_DEBUG=1 (libnvfp4kv_debug.so), every entry point also
// copies the device-side tables it trusts back to the host and range-checks
// them before launching anything.
#ifndef NVFP4KV_DEBUG
#define NVFP4KV_DEBUG 0
#endif
// Every check runs on the host before anything is queued; no exception
// crosses the interface and no device memory is allocated here.
#include "nvfp4kv.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <string>
#include <vector>

#include "nvfp4kv_internal.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Sizes and flags of the descriptor (the base pointer is not looked at).
int check_pool_shape(const nvfp4kv_pool* p) {
  if (p == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "pool descriptor is null");
  if (p->head_dim != 128) return fail(NVFP4KV_ERR_UNSUPPORTED, "head_dim %d unsupported (only 128)", p->head_dim);
  if (p->page_size != 64) return fail(NVFP4KV_ERR_UNSUPPORTED, "page_size %d unsupported (only 64)", p->page_size);
  if (p->num_pages <= 0) return fail(NVFP4KV_ERR_INVALID_ARG, "num_pages must be positive (got %lld)", (long long)p->num_pages);
  if (p->num_layers <= 0) return fail(NVFP4KV_ERR_INVALID_ARG, "num_layers must be positive (got %d)", p->num_layers);
  if (p->num_kv_heads <= 0) return fail(NVFP4KV_ERR_INVALID_ARG, "num_kv_heads must be positive (got %d)", p->num_kv_heads);
  if (p->rotary_dim < 0 || p->rotary_dim > 128 || p->rotary_dim % 2 != 0)
    return fail(NVFP4KV_ERR_INVALID_ARG, "rotary_dim %d invalid (even, 0..128)", p->rotary_dim);
  if (p->hadamard < 0 || p->hadamard > 2) return fail(NVFP4KV_ERR_INVALID_ARG, "hadamard must be 0, 1 or 2 (got %d)", p->hadamard);
  for (const float g : {p->k_scale, p->v_scale})
    if (g != 0.0f && !(g >= 0x1p-64f && g <= 0x1p64f))
      return fail(NVFP4KV_ERR_INVALID_ARG, "global scale %g out of range (0 = 1, else 2^-64..2^64)", (double)g);
  if (p->v_format != 0 && p->v_format != 1)
    return fail(NVFP4KV_ERR_INVALID_ARG, "v_format must be 0 (NVFP4 V) or 1 (fp16 V) (got %d)", p->v_format);
  return NVFP4KV_OK;
}

int check_pool(const nvfp4kv_pool* p) {
  int rc = check_pool_shape(p);
  if (rc != NVFP4KV_OK) return rc;
  if (p->base == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "pool base pointer is null");
  if (!aligned(p->base, 256)) return fail(NVFP4KV_ERR_INVALID_ARG, "pool base must be 256-byte aligned");
  return NVFP4KV_OK;
}

int check_layer(const nvfp4kv_pool* p, int32_t layer) {
  if (layer < 0 || layer >= p->num_layers)
    return fail(NVFP4KV_ERR_INVALID_ARG, "layer %d out of range [0, %d)", layer, p->num_layers);
  return NVFP4KV_OK;
}

int check_dtype(nvfp4kv_dtype d, const char* what) {
  if (d != NVFP4KV_F32 && d != NVFP4KV_BF16) return fail(NVFP4KV_ERR_INVALID_ARG, "%s dtype %d is not F32 or BF16", what, (int)d);
  return NVFP4KV_OK;
}

int check_rope(const nvfp4kv_pool* p, const float* c, const float* s, int32_t max_pos) {
  if (p->rotary_dim == 0) return NVFP4KV_OK;
  if (c == nullptr || s == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "rotary_dim > 0 needs rope_cos and rope_sin");
  if (max_pos <= 0) return fail(NVFP4KV_ERR_INVALID_ARG, "max_pos must be positive when rotary_dim > 0");
  if (!aligned(c, 16) || !aligned(s, 16)) return fail(NVFP4KV_ERR_INVALID_ARG, "rope_cos and rope_sin must be 16-byte aligned");
  return NVFP4KV_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(NVFP4KV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The decode kernels built for the pool's rotary width: multiples of 16
// (0 included) or the general rotation.
decltype(&nvfp4kv::launch_decode_splits) splits_launcher(const nvfp4kv_pool* p) {
  return (p->rotary_dim & 15) != 0 ? &nvfp4kv::launch_decode_splits_gr : &nvfp4kv::launch_decode_splits;
}

nvfp4kv::LaunchPool launch_pool(const nvfp4kv_pool* p) {
  nvfp4kv::LaunchPool L;
  L.base = reinterpret_cast<uint8_t*>(p->base);
  L.num_pages = p->num_pages;
  L.hkv = p->num_kv_heads;
  L.v_format = p->v_format;
  L.block_bytes = (int)nvfp4kv::pool_block_bytes(p->v_format);
  L.ks_off = nvfp4kv::pool_kscale_off(p->v_format);
  L.rotary_dim = p->rotary_dim;
  L.hadamard = p->hadamard;
  for (int i = 0; i < 4; ++i) L.signs.w[i] = p->hadamard == 2 ? p->hadamard_signs[i] : 0u;
  L.k_scale = p->k_scale == 0.0f ? 1.0f : p->k_scale;
  L.v_scale = p->v_scale == 0.0f ? 1.0f : p->v_scale;
  L.k_inv = 1.0f / L.k_scale;
  L.v_inv = 1.0f / L.v_scale;
  return L;
}

// Resident wavefronts of the decode kernels with `nt` column tiles (for one
// tile, packed groups or not) on the current device: CUs times one-wavefront
// workgroups per CU.  Cached per device (any thread may fill an entry; every
// thread computes the same value, so relaxed atomics suffice); if the device
// cannot be queried (no GPU), 256 CUs x 8 (one tile) or 4 (several tiles) is
// assumed so that size queries still work.
int resident_decode_waves(int nt, bool packed, bool vf16) {
  static std::atomic<int> cached[64][4][3];
  const int fallback = nt > 1 ? 256 * 4 : 256 * 8;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return fallback;
  }
  std::atomic<int>& slot = cached[dev][nt][vf16 ? 2 : packed ? 1 : 0];
  int c = slot.load(std::memory_order_relaxed);
  if (c == 0) {
    int cus = 0;
    const int per_cu = nvfp4kv::decode_waves_per_cu(nt, packed, vf16);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0 || per_cu <= 0) {
      (void)hipGetLastError();
      return fallback;
    }
    c = cus * per_cu;
    slot.store(c, std::memory_order_relaxed);
  }
  return c;
}

// Split-K plan.  The flattened (sequence, kv head, page) work is shared
// equally by n_waves one-wavefront workgroups.  pages_per_split 0 launches
// one wavefront per resident slot of the device; a positive value asks for
// about that many pages per wavefront at max_seq_len.  n_q_heads counts the
// query columns of the launch (query heads x new tokens), at most
// max_group per kv head.
int make_plan(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_q_heads, int64_t max_seq_len,
              int32_t pages_per_split, nvfp4kv::DecodePlan* out, int max_group = 16) {
  if (n_seq <= 0) return fail(NVFP4KV_ERR_INVALID_ARG, "n_seq must be positive (got %d)", n_seq);
  if (n_seq > 65535) return fail(NVFP4KV_ERR_UNSUPPORTED, "n_seq %d too large (at most 65535)", n_seq);
  if (n_q_heads <= 0 || n_q_heads % p->num_kv_heads != 0)
    return fail(NVFP4KV_ERR_INVALID_ARG, "n_q_heads %d must be a positive multiple of num_kv_heads %d", n_q_heads, p->num_kv_heads);
  const int group = n_q_heads / p->num_kv_heads;
  if (group > max_group) return fail(NVFP4KV_ERR_UNSUPPORTED, "%d query heads per kv head unsupported (at most %d)", group, max_group);
  if (max_seq_len <= 0) return fail(NVFP4KV_ERR_INVALID_ARG, "max_seq_len must be positive");
  const int64_t max_pages = (max_seq_len + 63) / 64;
  if (max_pages > ((int64_t)1 << 30)) return fail(NVFP4KV_ERR_INVALID_ARG, "max_seq_len too large");
  if (pages_per_split < 0 || pages_per_split > 4096)
    return fail(NVFP4KV_ERR_INVALID_ARG, "pages_per_split %d out of range (0 = automatic, else 1..4096)", pages_per_split);
  const int64_t max_total = (int64_t)n_seq * p->num_kv_heads * max_pages;
  int64_t waves;
  if (pages_per_split == 0)
    waves = resident_decode_waves(nvfp4kv::decode_column_tiles(group), group <= 8, p->v_format != 0);
  else
    waves = (max_total + pages_per_split - 1) / pages_per_split;
  waves = std::max<int64_t>(1, std::min<int64_t>(waves, std::min<int64_t>(max_total, (int64_t)1 << 24)));
  // the decode kernels count a wavefront's pages in 32 bits
  if ((max_total + (int64_t)5 * n_seq * p->num_kv_heads) / waves + 2 >= ((int64_t)1 << 30))
    return fail(NVFP4KV_ERR_UNSUPPORTED, "%lld pages over %lld wavefronts: too many pages per wavefront",
                (long long)max_total, (long long)waves);
  out->n_waves = (int)waves;
  out->group = group;
  return NVFP4KV_OK;
}

int check_workspace(size_t need, const void* workspace, size_t workspace_bytes) {
  if (workspace == nullptr || workspace_bytes < need)
    return fail(NVFP4KV_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(NVFP4KV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  return NVFP4KV_OK;
}

// ---- range checks of the device-side tables (on host copies) ----------------

int check_decode_tables_host(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_qtok, const int32_t* page_table,
                             int32_t page_table_stride, const int32_t* seq_lens, int64_t max_seq_len,
                             const int32_t* q_positions, int32_t max_pos) {
  int rc;
  if ((rc = check_pool_shape(p)) != NVFP4KV_OK) return rc;
  if (n_seq <= 0 || n_qtok <= 0) return fail(NVFP4KV_ERR_INVALID_ARG, "n_seq and n_qtok must be positive");
  if (page_table == nullptr || seq_lens == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "null page_table or seq_lens");
  if (max_seq_len <= 0 || page_table_stride < (max_seq_len + 63) / 64)
    return fail(NVFP4KV_ERR_INVALID_ARG, "page_table_stride %d smaller than the pages of max_seq_len %lld",
                page_table_stride, (long long)max_seq_len);
  for (int32_t n = 0; n < n_seq; ++n) {
    const int32_t L = seq_lens[n];
    if (L < n_qtok || (int64_t)L > max_seq_len)
      return fail(NVFP4KV_ERR_INVALID_ARG, "seq_lens[%d] = %d outside [%d, %lld]", n, L, n_qtok,
                  (long long)max_seq_len);
    for (int32_t j = 0; j < (L + 63) / 64; ++j) {
      const int32_t pid = page_table[(size_t)n * page_table_stride + j];
      if (pid < 0 || (int64_t)pid >= p->num_pages)
        return fail(NVFP4KV_ERR_INVALID_ARG, "page_table[%d][%d] = %d outside [0, %lld)", n, j, pid,
                    (long long)p->num_pages);
    }
  }
  if (p->rotary_dim > 0 && q_positions != nullptr)
    for (int64_t i = 0; i < (int64_t)n_seq * n_qtok; ++i)
      if (q_positions[i] < 0 || q_positions[i] >= max_pos)
        return fail(NVFP4KV_ERR_INVALID_ARG, "q_positions[%lld] = %d outside [0, %d)", (long long)i, q_positions[i],
                    max_pos);
  return NVFP4KV_OK;
}

int check_slots_host(const nvfp4kv_pool* p, int32_t n_tok, const int64_t* slots, const int32_t* positions,
                     int32_t max_pos) {
  int rc;
  if ((rc = check_pool_shape(p)) != NVFP4KV_OK) return rc;
  if (n_tok < 0) return fail(NVFP4KV_ERR_INVALID_ARG, "n_tok must not be negative");
  if (n_tok > 0 && slots == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "null slots");
  const int64_t n_slots = p->num_pages * 64;
  std::vector<std::pair<int64_t, int32_t>> order;
  order.reserve((size_t)n_tok);
  for (int32_t i = 0; i < n_tok; ++i) {
    if (slots[i] < 0 || slots[i] >= n_slots)
      return fail(NVFP4KV_ERR_INVALID_ARG, "slots[%d] = %lld outside [0, %lld)", i, (long long)slots[i],
                  (long long)n_slots);
    order.emplace_back(slots[i], i);
  }
  std::sort(order.begin(), order.end());
  for (size_t i = 1; i < order.size(); ++i)
    if (order[i].first == order[i - 1].first)
      return fail(NVFP4KV_ERR_INVALID_ARG, "slots[%d] and slots[%d] both name slot %lld (the writes would race)",
                  order[i - 1].second, order[i].second, (long long)order[i].first);
  if (p->rotary_dim > 0 && positions != nullptr)
    for (int32_t i = 0; i < n_tok; ++i)
      if (positions[i] < 0 || positions[i] >= max_pos)
        return fail(NVFP4KV_ERR_INVALID_ARG, "positions[%d] = %d outside [0, %d)", i, positions[i], max_pos);
  return NVFP4KV_OK;
}

int check_page_ids_host(const nvfp4kv_pool* p, int32_t n_pages, const int32_t* ids, int32_t distinct) {
  int rc;
  if ((rc = check_pool_shape(p)) != NVFP4KV_OK) return rc;
  if (n_pages < 0) return fail(NVFP4KV_ERR_INVALID_ARG, "n_pages must not be negative");
  if (n_pages > 0 && ids == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "null page ids");
  if (!distinct) return NVFP4KV_OK;   // ids outside the pool are skipped by contract
  std::vector<std::pair<int32_t, int32_t>> order;
  for (int32_t i = 0; i < n_pages; ++i)
    if (ids[i] >= 0 && (int64_t)ids[i] < p->num_pages) order.emplace_back(ids[i], i);
  std::sort(order.begin(), order.end());
  for (size_t i = 1; i < order.size(); ++i)
    if (order[i].first == order[i - 1].first)
      return fail(NVFP4KV_ERR_INVALID_ARG, "page_ids[%d] and page_ids[%d] both name page %d (a restore would mix them)",
                  order[i - 1].second, order[i].second, order[i].first);
  return NVFP4KV_OK;
}

#if NVFP4KV_DEBUG
// The checked build: copy the device-side tables a call trusts back to the
// host, in order on the call's stream, and range-check them before anything
// is launched.  This synchronizes the stream (a debugging aid only).
template <typename T>
int fetch(std::vector<T>& dst, const T* src, size_t n, hipStream_t stream) {
  dst.resize(n);
  if (n == 0) return NVFP4KV_OK;
  hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDefault, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "checked build: copying a table to the host");
  return NVFP4KV_OK;
}

int debug_check_decode(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_qtok, const int32_t* page_table,
                       int32_t stride, const int32_t* seq_lens, int64_t max_seq_len, const int32_t* q_positions,
                       int32_t max_pos, hipStream_t stream) {
  std::vector<int32_t> pt, sl, qp;
  int rc;
  if ((rc = fetch(sl, seq_lens, (size_t)n_seq, stream)) != NVFP4KV_OK) return rc;
  if ((rc = fetch(pt, page_table, (size_t)n_seq * stride, stream)) != NVFP4KV_OK) return rc;
  const bool pos = p->rotary_dim > 0 && q_positions != nullptr;
  if (pos && (rc = fetch(qp, q_positions, (size_t)n_seq * n_qtok, stream)) != NVFP4KV_OK) return rc;
  return check_decode_tables_host(p, n_seq, n_qtok, pt.data(), stride, sl.data(), max_seq_len,
                                  pos ? qp.data() : nullptr, max_pos);
}

int debug_check_slots(const nvfp4kv_pool* p, int32_t n_tok, const int64_t* slots, const int32_t* positions,
                      int32_t max_pos, hipStream_t stream) {
  std::vector<int64_t> sl;
  std::vector<int32_t> ps;
  int rc;
  if ((rc = fetch(sl, slots, (size_t)n_tok, stream)) != NVFP4KV_OK) return rc;
  const bool pos = p->rotary_dim > 0 && positions != nullptr;
  if (pos && (rc = fetch(ps, positions, (size_t)n_tok, stream)) != NVFP4KV_OK) return rc;
  return check_slots_host(p, n_tok, sl.data(), pos ? ps.data() : nullptr, max_pos);
}

int debug_check_page_ids(const nvfp4kv_pool* p, int32_t n_pages, const int32_t* ids, int32_t distinct,
                         hipStream_t stream) {
  std::vector<int32_t> v;
  int rc;
  if ((rc = fetch(v, ids, (size_t)n_pages, stream)) != NVFP4KV_OK) return rc;
  return check_page_ids_host(p, n_pages, v.data(), distinct);
}
#endif

}  // namespace

extern "C" {

int nvfp4kv_check_decode_tables(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_qtok, const int32_t* page_table,
                                int32_t page_table_stride, const int32_t* seq_lens, int64_t max_seq_len,
                                const int32_t* q_positions, int32_t max_pos) {
  g_last_error.clear();
  return check_decode_tables_host(p, n_seq, n_qtok, page_table, page_table_stride, seq_lens, max_seq_len,
                                  q_positions, max_pos);
}

int nvfp4kv_check_slots(const nvfp4kv_pool* p, int32_t n_tok, const int64_t* slots, const int32_t* positions,
                        int32_t max_pos) {
  g_last_error.clear();
  return check_slots_host(p, n_tok, slots, positions, max_pos);
}

int nvfp4kv_check_page_ids(const nvfp4kv_pool* p, int32_t n_pages, const int32_t* page_ids, int32_t distinct) {
  g_last_error.clear();
  return check_page_ids_host(p, n_pages, page_ids, distinct);
}

int nvfp4kv_checked_build(void) { return NVFP4KV_DEBUG ? 1 : 0; }

size_t nvfp4kv_pool_bytes(const nvfp4kv_pool* p) {
  if (p == nullptr || p->num_pages <= 0 || p->num_layers <= 0 || p->num_kv_heads <= 0 ||
      p->head_dim != 128 || p->page_size != 64 || (p->v_format != 0 && p->v_format != 1))
    return 0;
  return (size_t)p->num_layers * (size_t)p->num_pages * (size_t)p->num_kv_heads *
         nvfp4kv::pool_block_bytes(p->v_format);
}

int nvfp4kv_rope_table(double theta, int32_t rotary_dim, double pos_scale, int32_t max_pos,
                       float* cos_out, float* sin_out) {
  g_last_error.clear();
  if (cos_out == nullptr || sin_out == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "null output table");
  if (rotary_dim <= 0 || rotary_dim > 128 || rotary_dim % 2 != 0) return fail(NVFP4KV_ERR_INVALID_ARG, "rotary_dim %d invalid", rotary_dim);
  if (max_pos <= 0) return fail(NVFP4KV_ERR_INVALID_ARG, "max_pos must be positive");
  if (!(theta > 0.0) || !(pos_scale > 0.0)) return fail(NVFP4KV_ERR_INVALID_ARG, "theta and pos_scale must be positive");
  const int half = rotary_dim / 2;
  for (int32_t pos = 0; pos < max_pos; ++pos) {
    for (int i = 0; i < half; ++i) {
      const double inv = pow(theta, -(2.0 * i) / (double)rotary_dim);
      const double ang = ((double)pos / pos_scale) * inv;
      cos_out[(size_t)pos * half + i] = (float)cos(ang);
      sin_out[(size_t)pos * half + i] = (float)sin(ang);
    }
  }
  return NVFP4KV_OK;
}

int nvfp4kv_append(const nvfp4kv_pool* p, int32_t layer, int32_t n_tok, const void* k,
                   const void* v, nvfp4kv_dtype in_dtype, const int64_t* slots,
                   const int32_t* positions, const float* rope_cos, const float* rope_sin,
                   int32_t max_pos, hipStream_t stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_pool(p)) != NVFP4KV_OK) return rc;
  if ((rc = check_layer(p, layer)) != NVFP4KV_OK) return rc;
  if ((rc = check_dtype(in_dtype, "input")) != NVFP4KV_OK) return rc;
  if (n_tok < 0) return fail(NVFP4KV_ERR_INVALID_ARG, "n_tok must not be negative (got %d)", n_tok);
  if (n_tok == 0) return NVFP4KV_OK;
  if ((int64_t)n_tok * p->num_kv_heads * 2 > (int64_t)1 << 30) return fail(NVFP4KV_ERR_UNSUPPORTED, "too many rows in one append");
  if (k == nullptr || v == nullptr || slots == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "null k, v or slots");
  if (!aligned(k, 16) || !aligned(v, 16)) return fail(NVFP4KV_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if (p->rotary_dim > 0 && positions == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "rotary_dim > 0 needs positions");
  if ((rc = check_rope(p, rope_cos, rope_sin, max_pos)) != NVFP4KV_OK) return rc;
#if NVFP4KV_DEBUG
  if ((rc = debug_check_slots(p, n_tok, slots, positions, max_pos, stream)) != NVFP4KV_OK) return rc;
#endif
  hipError_t e = nvfp4kv::launch_append(launch_pool(p), layer, n_tok, k, v, (int)in_dtype, slots,
                                        positions, rope_cos, rope_sin, stream);
  if (e != hipSuccess) return hip_fail(e, "kv_quant_append launch");
  return NVFP4KV_OK;
}

size_t nvfp4kv_decode_workspace_bytes(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_q_heads,
                                      int64_t max_seq_len, int32_t pages_per_split) {
  g_last_error.clear();
  if (check_pool_shape(p) != NVFP4KV_OK) return 0;
  nvfp4kv::DecodePlan plan;
  if (make_plan(p, n_seq, n_q_heads, max_seq_len, pages_per_split, &plan) != NVFP4KV_OK) return 0;
  return nvfp4kv::ws_bytes(n_seq, p->num_kv_heads, plan);
}

// The one new query token of a plain decode call.
static nvfp4kv::QTokens one_token(const nvfp4kv::DecodePlan& plan) {
  return nvfp4kv::QTokens{1, 0, plan.group};
}

// Query tokens per launch of a multi-token decode: as many as fit the
// kernel's 48 columns with every query head of a kv head (at least 1).
static int tokens_per_launch(int heads, int n_qtok) {
  return std::max(1, std::min(n_qtok, nvfp4kv::kMaxDecodeColumns / heads));
}

// Checks shared by the decode entry points; fills `plan`.
static int check_decode(const nvfp4kv_pool* p, int32_t layer, int32_t n_seq, int32_t n_q_heads,
                        const void* q, const void* k_new, const void* v_new,
                        nvfp4kv_dtype q_dtype, const int32_t* q_positions,
                        const float* rope_cos, const float* rope_sin, int32_t max_pos,
                        const int32_t* page_table, int32_t page_table_stride,
                        const int32_t* seq_lens, int64_t max_seq_len, float sm_scale,
                        const void* workspace, size_t workspace_bytes, int32_t pages_per_split,
                        nvfp4kv::DecodePlan* plan, int max_group = 16) {
  int rc;
  if ((rc = check_pool(p)) != NVFP4KV_OK) return rc;
  if ((rc = check_layer(p, layer)) != NVFP4KV_OK) return rc;
  if ((rc = check_dtype(q_dtype, "query")) != NVFP4KV_OK) return rc;
  if ((rc = make_plan(p, n_seq, n_q_heads, max_seq_len, pages_per_split, plan, max_group)) != NVFP4KV_OK) return rc;
  if (p->v_format == 1 && plan->group > 8)
    return fail(NVFP4KV_ERR_UNSUPPORTED, "fp16 V (v_format 1) takes up to 8 query heads per kv head (got %d)",
                plan->group);
  if (q == nullptr || page_table == nullptr || seq_lens == nullptr)
    return fail(NVFP4KV_ERR_INVALID_ARG, "null q, page_table or seq_lens");
  if (!aligned(q, 16)) return fail(NVFP4KV_ERR_INVALID_ARG, "q must be 16-byte aligned");
  if ((k_new == nullptr) != (v_new == nullptr))
    return fail(NVFP4KV_ERR_INVALID_ARG, "k_new and v_new must both be given or both be null");
  if (k_new != nullptr && (!aligned(k_new, 16) || !aligned(v_new, 16)))
    return fail(NVFP4KV_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  if (p->rotary_dim > 0 && q_positions == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "rotary_dim > 0 needs q_positions");
  if ((rc = check_rope(p, rope_cos, rope_sin, max_pos)) != NVFP4KV_OK) return rc;
  const int64_t max_pages = (max_seq_len + 63) / 64;
  if (page_table_stride < max_pages)
    return fail(NVFP4KV_ERR_INVALID_ARG, "page_table_stride %d smaller than the %lld pages of max_seq_len", page_table_stride, (long long)max_pages);
  if (!(sm_scale >= 0.0f) || !isfinite(sm_scale)) return fail(NVFP4KV_ERR_INVALID_ARG, "sm_scale must be finite and >= 0");
  return check_workspace(nvfp4kv::ws_bytes(n_seq, p->num_kv_heads, *plan), workspace, workspace_bytes);
}

int nvfp4kv_decode_attn_splits(const nvfp4kv_pool* p, int32_t layer, int32_t n_seq,
                               int32_t n_q_heads, const void* q, const void* k_new,
                               const void* v_new, nvfp4kv_dtype q_dtype,
                               const int32_t* q_positions, const float* rope_cos,
                               const float* rope_sin, int32_t max_pos, const int32_t* page_table,
                               int32_t page_table_stride, const int32_t* seq_lens,
                               int64_t max_seq_len, float sm_scale, void* workspace,
                               size_t workspace_bytes, int32_t pages_per_split, hipStream_t stream) {
  g_last_error.clear();
  nvfp4kv::DecodePlan plan;
  int rc = check_decode(p, layer, n_seq, n_q_heads, q, k_new, v_new, q_dtype, q_positions, rope_cos, rope_sin,
                        max_pos, page_table, page_table_stride, seq_lens, max_seq_len, sm_scale,
                        workspace, workspace_bytes, pages_per_split, &plan);
  if (rc != NVFP4KV_OK) return rc;
#if NVFP4KV_DEBUG
  if ((rc = debug_check_decode(p, n_seq, 1, page_table, page_table_stride, seq_lens, max_seq_len, q_positions,
                               max_pos, stream)) != NVFP4KV_OK)
    return rc;
#endif
  hipError_t e = splits_launcher(p)(launch_pool(p), layer, n_seq, n_q_heads, q, k_new,
                                               v_new, (int)q_dtype, q_positions, rope_cos, rope_sin,
                                               page_table, page_table_stride, seq_lens, sm_scale,
                                               workspace, plan, one_token(plan), stream);
  if (e != hipSuccess) return hip_fail(e, "decode_attn_splitk launch");
  return NVFP4KV_OK;
}

int nvfp4kv_decode_reduce(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_q_heads,
                          const int32_t* seq_lens, int64_t max_seq_len, float* out,
                          const void* workspace, size_t workspace_bytes, int32_t pages_per_split,
                          hipStream_t stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_pool_shape(p)) != NVFP4KV_OK) return rc;
  nvfp4kv::DecodePlan plan;
  if ((rc = make_plan(p, n_seq, n_q_heads, max_seq_len, pages_per_split, &plan)) != NVFP4KV_OK) return rc;
  if (seq_lens == nullptr || out == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "null seq_lens or out");
  if (!aligned(out, 16)) return fail(NVFP4KV_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if ((rc = check_workspace(nvfp4kv::ws_bytes(n_seq, p->num_kv_heads, plan), workspace, workspace_bytes)) != NVFP4KV_OK) return rc;
  hipError_t e = nvfp4kv::launch_decode_reduce(p->num_kv_heads, n_seq, n_q_heads, seq_lens, out,
                                               workspace, plan, one_token(plan), launch_pool(p).v_scale, stream);
  if (e != hipSuccess) return hip_fail(e, "decode_reduce launch");
  return NVFP4KV_OK;
}

int nvfp4kv_decode_attn(const nvfp4kv_pool* p, int32_t layer, int32_t n_seq, int32_t n_q_heads,
                        const void* q, const void* k_new, const void* v_new,
                        nvfp4kv_dtype q_dtype, const int32_t* q_positions,
                        const float* rope_cos, const float* rope_sin, int32_t max_pos,
                        const int32_t* page_table, int32_t page_table_stride,
                        const int32_t* seq_lens, int64_t max_seq_len, float sm_scale, float* out,
                        void* workspace, size_t workspace_bytes, int32_t pages_per_split,
                        hipStream_t stream) {
  g_last_error.clear();
  nvfp4kv::DecodePlan plan;
  int rc = check_decode(p, layer, n_seq, n_q_heads, q, k_new, v_new, q_dtype, q_positions, rope_cos, rope_sin,
                        max_pos, page_table, page_table_stride, seq_lens, max_seq_len, sm_scale,
                        workspace, workspace_bytes, pages_per_split, &plan);
  if (rc != NVFP4KV_OK) return rc;
  if (out == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "null out");
  if (!aligned(out, 16)) return fail(NVFP4KV_ERR_INVALID_ARG, "out must be 16-byte aligned");
#if NVFP4KV_DEBUG
  if ((rc = debug_check_decode(p, n_seq, 1, page_table, page_table_stride, seq_lens, max_seq_len, q_positions,
                               max_pos, stream)) != NVFP4KV_OK)
    return rc;
#endif
  hipError_t e = splits_launcher(p)(launch_pool(p), layer, n_seq, n_q_heads, q, k_new,
                                               v_new, (int)q_dtype, q_positions, rope_cos, rope_sin,
                                               page_table, page_table_stride, seq_lens, sm_scale,
                                               workspace, plan, one_token(plan), stream);
  if (e != hipSuccess) return hip_fail(e, "decode_attn_splitk launch");
  e = nvfp4kv::launch_decode_reduce(p->num_kv_heads, n_seq, n_q_heads, seq_lens, out, workspace,
                                    plan, one_token(plan), launch_pool(p).v_scale, stream);
  if (e != hipSuccess) return hip_fail(e, "decode_reduce launch");
  return NVFP4KV_OK;
}

int nvfp4kv_decode_attn_static(const nvfp4kv_pool* p, int32_t layer, int32_t n_seq, int32_t n_q_heads,
                               const void* q, const void* k_new, const void* v_new,
                               nvfp4kv_dtype q_dtype, const int32_t* q_positions,
                               const float* rope_cos, const float* rope_sin, int32_t max_pos,
                               const int32_t* page_table, int32_t page_table_stride,
                               const int32_t* seq_lens, int64_t max_seq_len, float sm_scale, float* out,
                               int32_t pages_per_split, hipStream_t stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_pool(p)) != NVFP4KV_OK) return rc;
  nvfp4kv::DecodePlan plan;
  if ((rc = make_plan(p, n_seq, n_q_heads, max_seq_len, pages_per_split, &plan)) != NVFP4KV_OK) return rc;
  const size_t need = nvfp4kv::ws_bytes(n_seq, p->num_kv_heads, plan);
  if (need > nvfp4kv::kStaticWorkspaceBytes)
    return fail(NVFP4KV_ERR_WORKSPACE,
                "this decode needs %zu workspace bytes, more than the %zu of the static workspace "
                "(use nvfp4kv_decode_attn with a caller-allocated workspace)",
                need, nvfp4kv::kStaticWorkspaceBytes);
  void* ws = nullptr;
  hipError_t e = nvfp4kv::static_workspace(&ws);
  if (e != hipSuccess) return hip_fail(e, "static workspace address");
  return nvfp4kv_decode_attn(p, layer, n_seq, n_q_heads, q, k_new, v_new, q_dtype, q_positions, rope_cos,
                             rope_sin, max_pos, page_table, page_table_stride, seq_lens, max_seq_len, sm_scale,
                             out, ws, nvfp4kv::kStaticWorkspaceBytes, pages_per_split, stream);
}

// Shape checks of a multi-token decode; `cols` = query columns per launch.
static int check_multi_shape(const nvfp4kv_pool* p, int32_t n_qtok, int32_t n_q_heads, int* cols,
                             int* per_launch) {
  if (n_qtok < 1 || n_qtok > 64)
    return fail(NVFP4KV_ERR_INVALID_ARG, "n_qtok %d out of range (1..64)", n_qtok);
  if (n_q_heads <= 0 || n_q_heads % p->num_kv_heads != 0)
    return fail(NVFP4KV_ERR_INVALID_ARG, "n_q_heads %d must be a positive multiple of num_kv_heads %d", n_q_heads, p->num_kv_heads);
  const int heads = n_q_heads / p->num_kv_heads;
  if (heads > 16) return fail(NVFP4KV_ERR_UNSUPPORTED, "%d query heads per kv head unsupported (at most 16)", heads);
  *per_launch = tokens_per_launch(heads, n_qtok);
  *cols = *per_launch * heads;
  return NVFP4KV_OK;
}

// Plans of the launches of a multi-token decode: every launch takes `per`
// tokens but the last, which takes the rest; the workspace is reused in
// stream order, so it must hold the larger of the two plans' partials.
static int multi_plans(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_qtok, int heads, int per,
                       int64_t max_seq_len, int32_t pages_per_split, nvfp4kv::DecodePlan* full,
                       nvfp4kv::DecodePlan* last, size_t* need) {
  const int hkv = p->num_kv_heads;
  int rc = make_plan(p, n_seq, hkv * per * heads, max_seq_len, pages_per_split, full,
                     nvfp4kv::kMaxDecodeColumns);
  if (rc != NVFP4KV_OK) return rc;
  const int rest = n_qtok % per == 0 ? per : n_qtok % per;
  rc = make_plan(p, n_seq, hkv * rest * heads, max_seq_len, pages_per_split, last, nvfp4kv::kMaxDecodeColumns);
  if (rc != NVFP4KV_OK) return rc;
  *need = std::max(nvfp4kv::ws_bytes(n_seq, hkv, *full), nvfp4kv::ws_bytes(n_seq, hkv, *last));
  return NVFP4KV_OK;
}

size_t nvfp4kv_decode_multi_workspace_bytes(const nvfp4kv_pool* p, int32_t n_seq, int32_t n_qtok,
                                            int32_t n_q_heads, int64_t max_seq_len,
                                            int32_t pages_per_split) {
  g_last_error.clear();
  if (check_pool_shape(p) != NVFP4KV_OK) return 0;
  int cols = 0, per = 0;
  if (check_multi_shape(p, n_qtok, n_q_heads, &cols, &per) != NVFP4KV_OK) return 0;
  nvfp4kv::DecodePlan full, last;
  size_t need = 0;
  if (multi_plans(p, n_seq, n_qtok, n_q_heads / p->num_kv_heads, per, max_seq_len, pages_per_split, &full,
                  &last, &need) != NVFP4KV_OK)
    return 0;
  return need;
}

int nvfp4kv_decode_attn_multi(const nvfp4kv_pool* p, int32_t layer, int32_t n_seq, int32_t n_qtok,
                              int32_t n_q_heads, const void* q, nvfp4kv_dtype q_dtype,
                              const int32_t* q_positions, const float* rope_cos,
                              const float* rope_sin, int32_t max_pos, const int32_t* page_table,
                              int32_t page_table_stride, const int32_t* seq_lens,
                              int64_t max_seq_len, float sm_scale, float* out, void* workspace,
                              size_t workspace_bytes, int32_t pages_per_split, hipStream_t stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_pool(p)) != NVFP4KV_OK) return rc;
  if (p->v_format != 0)
    return fail(NVFP4KV_ERR_UNSUPPORTED, "multi-token decode reads NVFP4 V only (v_format 0)");
  int cols = 0, per = 0;
  if ((rc = check_multi_shape(p, n_qtok, n_q_heads, &cols, &per)) != NVFP4KV_OK) return rc;
  nvfp4kv::DecodePlan full, last;
  rc = check_decode(p, layer, n_seq, p->num_kv_heads * cols, q, nullptr, nullptr, q_dtype, q_positions,
                    rope_cos, rope_sin, max_pos, page_table, page_table_stride, seq_lens, max_seq_len,
                    sm_scale, workspace, workspace_bytes, pages_per_split, &full, nvfp4kv::kMaxDecodeColumns);
  if (rc != NVFP4KV_OK) return rc;
  if (out == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "null out");
  if (!aligned(out, 16)) return fail(NVFP4KV_ERR_INVALID_ARG, "out must be 16-byte aligned");
  const int heads = n_q_heads / p->num_kv_heads;
  size_t need = 0;
  if ((rc = multi_plans(p, n_seq, n_qtok, heads, per, max_seq_len, pages_per_split, &full, &last, &need)) !=
      NVFP4KV_OK)
    return rc;
  if ((rc = check_workspace(need, workspace, workspace_bytes)) != NVFP4KV_OK) return rc;
#if NVFP4KV_DEBUG
  if ((rc = debug_check_decode(p, n_seq, n_qtok, page_table, page_table_stride, seq_lens, max_seq_len, q_positions,
                               max_pos, stream)) != NVFP4KV_OK)
    return rc;
#endif
  // one split + reduce pair per launch's tokens; the workspace is reused in
  // stream order
  for (int t0 = 0; t0 < n_qtok; t0 += per) {
    const nvfp4kv::DecodePlan& pl = t0 + per <= n_qtok ? full : last;
    const nvfp4kv::QTokens qt{n_qtok, t0, heads};
    hipError_t e = splits_launcher(p)(launch_pool(p), layer, n_seq, n_q_heads, q, nullptr, nullptr,
                                                 (int)q_dtype, q_positions, rope_cos, rope_sin, page_table,
                                                 page_table_stride, seq_lens, sm_scale, workspace, pl, qt,
                                                 stream);
    if (e != hipSuccess) return hip_fail(e, "decode_attn_splitk launch");
    e = nvfp4kv::launch_decode_reduce(p->num_kv_heads, n_seq, n_q_heads, seq_lens, out, workspace, pl,
                                      qt, launch_pool(p).v_scale, stream);
    if (e != hipSuccess) return hip_fail(e, "decode_reduce launch");
  }
  return NVFP4KV_OK;
}

size_t nvfp4kv_page_bytes(const nvfp4kv_pool* p) {
  g_last_error.clear();
  if (check_pool_shape(p) != NVFP4KV_OK) return 0;
  return (size_t)p->num_layers * (size_t)p->num_kv_heads * nvfp4kv::pool_block_bytes(p->v_format);
}

// Device address at which kernels reach `ptr`: device memory of the current
// device as is, pinned host memory through its device mapping.  Anything
// else (pageable host memory, another device's memory) is refused before any
// launch, since a kernel access to it would fault.
static int device_view(const void* ptr, const char* what, uint8_t** out) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, ptr) != hipSuccess) {
    (void)hipGetLastError();
    return fail(NVFP4KV_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", what);
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return hip_fail(hipGetLastError(), "hipGetDevice");
  if (at.type == hipMemoryTypeDevice) {
    if (at.device != dev) return fail(NVFP4KV_ERR_INVALID_ARG, "%s is memory of device %d, not of the current device %d", what, at.device, dev);
    *out = const_cast<uint8_t*>(static_cast<const uint8_t*>(ptr));
    return NVFP4KV_OK;
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer != nullptr && at.hostPointer != nullptr) {
    *out = static_cast<uint8_t*>(at.devicePointer) +
           (static_cast<const uint8_t*>(ptr) - static_cast<const uint8_t*>(at.hostPointer));
    return NVFP4KV_OK;
  }
  return fail(NVFP4KV_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", what);
}

static int page_copy(const nvfp4kv_pool* p, int32_t n_pages, const int32_t* page_ids, const void* arena,
                     size_t arena_bytes, bool to_arena, hipStream_t stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_pool(p)) != NVFP4KV_OK) return rc;
  if (n_pages < 0) return fail(NVFP4KV_ERR_INVALID_ARG, "n_pages must not be negative (got %d)", n_pages);
  if (n_pages == 0) return NVFP4KV_OK;
  if (page_ids == nullptr || arena == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "null page_ids or arena");
  if (!aligned(arena, 16)) return fail(NVFP4KV_ERR_INVALID_ARG, "arena must be 16-byte aligned");
  const size_t page = (size_t)p->num_layers * (size_t)p->num_kv_heads * nvfp4kv::pool_block_bytes(p->v_format);
  if (arena_bytes / page < (size_t)n_pages)
    return fail(NVFP4KV_ERR_INVALID_ARG, "arena of %zu bytes holds fewer than %d pages of %zu bytes", arena_bytes, n_pages, page);
  uint8_t* ids_dev = nullptr;
  uint8_t* arena_dev = nullptr;
  if ((rc = device_view(page_ids, "page_ids", &ids_dev)) != NVFP4KV_OK) return rc;
  if ((rc = device_view(arena, "arena", &arena_dev)) != NVFP4KV_OK) return rc;
#if NVFP4KV_DEBUG
  if ((rc = debug_check_page_ids(p, n_pages, page_ids, to_arena ? 0 : 1, stream)) != NVFP4KV_OK) return rc;
#endif
  hipError_t e = nvfp4kv::launch_page_copy(launch_pool(p), p->num_layers, n_pages,
                                           reinterpret_cast<const int32_t*>(ids_dev), arena_dev, to_arena, stream);
  if (e != hipSuccess) return hip_fail(e, "page copy launch");
  return NVFP4KV_OK;
}

int nvfp4kv_spill_pages(const nvfp4kv_pool* p, int32_t n_pages, const int32_t* page_ids, void* arena,
                        size_t arena_bytes, hipStream_t stream) {
  return page_copy(p, n_pages, page_ids, arena, arena_bytes, true, stream);
}

int nvfp4kv_restore_pages(const nvfp4kv_pool* p, int32_t n_pages, const int32_t* page_ids,
                          const void* arena, size_t arena_bytes, hipStream_t stream) {
  return page_copy(p, n_pages, page_ids, arena, arena_bytes, false, stream);
}

int nvfp4kv_stream_read(const nvfp4kv_pool* p, int32_t layer, int32_t n_seq, const int32_t* page_table,
                        int32_t page_table_stride, const int32_t* seq_lens, int32_t n_waves, uint32_t* words,
                        hipStream_t stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_pool(p)) != NVFP4KV_OK) return rc;
  if ((rc = check_layer(p, layer)) != NVFP4KV_OK) return rc;
  if (n_seq <= 0) return fail(NVFP4KV_ERR_INVALID_ARG, "n_seq must be positive (got %d)", n_seq);
  if (p->v_format != 0) return fail(NVFP4KV_ERR_UNSUPPORTED, "the read probe covers NVFP4 pools (v_format 0) only");
  if (n_waves <= 0 || n_waves > (1 << 24)) return fail(NVFP4KV_ERR_INVALID_ARG, "n_waves %d out of range (1..2^24)", n_waves);
  if (page_table == nullptr || seq_lens == nullptr || words == nullptr)
    return fail(NVFP4KV_ERR_INVALID_ARG, "null page_table, seq_lens or words");
  if (page_table_stride <= 0) return fail(NVFP4KV_ERR_INVALID_ARG, "page_table_stride must be positive");
  hipError_t e = nvfp4kv::launch_stream_read(launch_pool(p), layer, n_seq, page_table, page_table_stride,
                                             seq_lens, n_waves, words, stream);
  if (e != hipSuccess) return hip_fail(e, "stream_read launch");
  return NVFP4KV_OK;
}

int nvfp4kv_dequant(const nvfp4kv_pool* p, int32_t layer, int32_t n_tok, const int64_t* slots,
                    void* k_out, void* v_out, nvfp4kv_dtype out_dtype, int32_t unrotate,
                    hipStream_t stream) {
  g_last_error.clear();
  int rc;
  if ((rc = check_pool(p)) != NVFP4KV_OK) return rc;
  if ((rc = check_layer(p, layer)) != NVFP4KV_OK) return rc;
  if ((rc = check_dtype(out_dtype, "output")) != NVFP4KV_OK) return rc;
  if (n_tok < 0) return fail(NVFP4KV_ERR_INVALID_ARG, "n_tok must not be negative (got %d)", n_tok);
  if (n_tok == 0) return NVFP4KV_OK;
  if ((int64_t)n_tok * p->num_kv_heads * 2 > (int64_t)1 << 30) return fail(NVFP4KV_ERR_UNSUPPORTED, "too many rows in one dequant");
  if (slots == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "null slots");
  if (k_out == nullptr && v_out == nullptr) return fail(NVFP4KV_ERR_INVALID_ARG, "k_out and v_out are both null");
  if ((k_out && !aligned(k_out, 16)) || (v_out && !aligned(v_out, 16)))
    return fail(NVFP4KV_ERR_INVALID_ARG, "outputs must be 16-byte aligned");
  if (unrotate != 0 && unrotate != 1) return fail(NVFP4KV_ERR_INVALID_ARG, "unrotate must be 0 or 1");
#if NVFP4KV_DEBUG
  {
    // reads may repeat a slot: only the range is checked
    std::vector<int64_t> sl;
    if ((rc = fetch(sl, slots, (size_t)n_tok, stream)) != NVFP4KV_OK) return rc;
    for (int32_t i = 0; i < n_tok; ++i)
      if (sl[i] < 0 || sl[i] >= p->num_pages * 64)
        return fail(NVFP4KV_ERR_INVALID_ARG, "slots[%d] = %lld outside [0, %lld)", i, (long long)sl[i],
                    (long long)(p->num_pages * 64));
  }
#endif
  hipError_t e = nvfp4kv::launch_dequant(launch_pool(p), layer, n_tok, slots, k_out, v_out,
                                         (int)out_dtype, unrotate, stream);
  if (e != hipSuccess) return hip_fail(e, "dequant launch");
  return NVFP4KV_OK;
}

const char* nvfp4kv_last_error(void) { return g_last_error.c_str(); }

const char* nvfp4kv_version(void) { return "nvfp4kv 0.1.0 gfx950"; }

}  // extern "C"
