// libdsa C ABI: argument validation, workspace layout and kernel dispatch.
// Every check runs on the host before anything is enqueued, so a rejected
// call has no side effect on the device.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>

#include "dsa.h"
#include "dsa_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t n_blocks(const dsa_shape* s) { return ((int64_t)s->seq_len + s->block - 1) / s->block; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// common shape checks; decode adds its own
int check_shape(const dsa_shape* s) {
  if (!s) return fail(DSA_ERR_NULL, "shape is NULL");
  if (s->batch < 0) return fail(DSA_ERR_SHAPE, "batch %d < 0", s->batch);
  if (s->seq_len < 0) return fail(DSA_ERR_SHAPE, "seq_len %d < 0", s->seq_len);
  if (s->n_q_heads < 1 || s->n_kv_heads < 1)
    return fail(DSA_ERR_SHAPE, "head counts must be >= 1 (Hq %d, Hkv %d)", s->n_q_heads, s->n_kv_heads);
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(DSA_ERR_SHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d", s->n_q_heads, s->n_kv_heads);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "head_dim %d (built: 64, 128)", s->head_dim);
  if (s->block != 64 && s->block != 128) return fail(DSA_ERR_UNSUPPORTED, "block %d (built: 64, 128)", s->block);
  if (s->topk < 0) return fail(DSA_ERR_SHAPE, "topk %d < 0", s->topk);
  if (s->flags & ~(DSA_FORCE_SINK | DSA_FORCE_DIAG | DSA_DETERMINISTIC))
    return fail(DSA_ERR_SHAPE, "unknown flags 0x%x", s->flags);
  const uint32_t forced = s->flags & (DSA_FORCE_SINK | DSA_FORCE_DIAG);
  if (s->select_mode != DSA_SELECT_TOPK && s->select_mode != DSA_SELECT_THRESHOLD &&
      s->select_mode != DSA_SELECT_ENTROPY)
    return fail(DSA_ERR_SHAPE, "unknown select_mode %d", s->select_mode);
  if (s->n_anchor < 0 || s->window < 0)
    return fail(DSA_ERR_SHAPE, "n_anchor %d and window %d must be >= 0", s->n_anchor, s->window);
  if (s->select_mode == DSA_SELECT_THRESHOLD && !(s->threshold > 0.f && s->threshold <= 1.f))
    return fail(DSA_ERR_SHAPE, "threshold %g is not in (0, 1]", (double)s->threshold);
  if (s->select_mode == DSA_SELECT_THRESHOLD && forced == 0)
    return fail(DSA_ERR_SHAPE, "threshold selection needs a forced block (a row could keep none)");
  if (s->select_mode == DSA_SELECT_ENTROPY && !(s->k_min >= 1 && s->k_min <= s->k_max))
    return fail(DSA_ERR_SHAPE, "entropy budget needs 1 <= k_min (%d) <= k_max (%d)", s->k_min, s->k_max);
  if (s->select_mode == DSA_SELECT_TOPK && s->topk == 0) {
    if (s->topk_den < 1) return fail(DSA_ERR_SHAPE, "topk_den %d < 1", s->topk_den);
    if (s->topk_num < 0) return fail(DSA_ERR_SHAPE, "topk_num %d < 0", s->topk_num);
    if (s->topk_num == 0 && forced == 0)
      return fail(DSA_ERR_SHAPE, "topk, topk_num and the forcing flags are all 0: no block kept");
  }
  if (n_blocks(s) > DSA_MAX_BLOCKS)
    return fail(DSA_ERR_UNSUPPORTED, "%lld blocks > %d", (long long)n_blocks(s), DSA_MAX_BLOCKS);
  // grid sizes must fit the 32-bit launch dimensions
  const int64_t units = (int64_t)s->batch * std::max(s->n_q_heads, s->n_kv_heads);
  if (units * n_blocks(s) >= (1ll << 31)) return fail(DSA_ERR_UNSUPPORTED, "problem too large for one launch");
  return DSA_OK;
}

int check_decode(const dsa_shape* s) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (s->batch > 0 && s->seq_len < 1) return fail(DSA_ERR_SHAPE, "decode needs a cache of at least 1 position");
  if (s->select_mode != DSA_SELECT_TOPK)
    return fail(DSA_ERR_UNSUPPORTED, "decode selects by top-k only (select_mode %d)", s->select_mode);
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(DSA_ERR_UNSUPPORTED, "decode group size %d (built: 1, 2, 4, 8)", G);
  return DSA_OK;
}

int anchors_of(const dsa_shape* s) { return (s->flags & DSA_FORCE_SINK) ? std::max(1, s->n_anchor) : 0; }
int window_of(const dsa_shape* s) { return (s->flags & DSA_FORCE_DIAG) ? std::max(1, s->window) : 0; }

// forced blocks of a row that sees `visible` blocks: a prefix of anchors and
// a suffix (the window), overlapping when the row is short
int n_forced(const dsa_shape* s, int visible) {
  const int na = std::min(anchors_of(s), visible);
  const int ws = std::max(visible - window_of(s), na);
  return na + (visible - ws);
}

// most candidates a threshold row can keep: their shares sum to <= 1
int cand_cap(const dsa_shape* s) {
  if (s->select_mode != DSA_SELECT_THRESHOLD) return 0;
  return (int)std::min(floor(1.0 / (double)s->threshold), (double)DSA_MAX_BLOCKS);
}

// most blocks a row that sees `visible` blocks keeps
int row_budget(const dsa_shape* s, int visible) {
  const int nf = n_forced(s, visible);
  int64_t k;
  if (s->select_mode == DSA_SELECT_THRESHOLD) k = (int64_t)nf + cand_cap(s);
  else if (s->select_mode == DSA_SELECT_ENTROPY) k = s->k_max;
  else k = s->topk > 0 ? s->topk : ((int64_t)s->topk_num * visible + s->topk_den - 1) / s->topk_den;
  k = std::max<int64_t>(k, nf);
  k = std::min<int64_t>(k, visible);
  return (int)k;
}

int prefill_kmax(const dsa_shape* s) {
  int best = 0;
  for (int i = 0; i < n_blocks(s); ++i) best = std::max(best, row_budget(s, i + 1));
  return best;
}

dsa::TopkParams topk_params(const dsa_shape* s) {
  return dsa::TopkParams{s->topk,         s->topk_num,       s->topk_den, s->flags, anchors_of(s), window_of(s),
                         s->select_mode, s->threshold, s->k_min,    s->k_max, cand_cap(s)};
}

bool empty_prefill(const dsa_shape* s) { return s->batch == 0 || s->seq_len == 0; }

int check_index(const dsa_index_shape* s) {
  if (!s) return fail(DSA_ERR_NULL, "shape is NULL");
  if (s->batch < 0) return fail(DSA_ERR_SHAPE, "batch %d < 0", s->batch);
  if (s->seq_len < 0) return fail(DSA_ERR_SHAPE, "seq_len %d < 0", s->seq_len);
  if (s->n_q_heads < 1 || s->n_kv_heads < 1 || s->n_q_heads % s->n_kv_heads != 0)
    return fail(DSA_ERR_SHAPE, "head counts Hq %d, Hkv %d", s->n_q_heads, s->n_kv_heads);
  const int G = s->n_q_heads / s->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(DSA_ERR_UNSUPPORTED, "group size %d (built: 1, 2, 4, 8)", G);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "head_dim %d (built: 64, 128)", s->head_dim);
  if (s->n_index_heads != DSA_INDEX_HEADS)
    return fail(DSA_ERR_UNSUPPORTED, "n_index_heads %d (built: %d)", s->n_index_heads, DSA_INDEX_HEADS);
  if (s->index_dim != 64 && s->index_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "index_dim %d (built: 64, 128)", s->index_dim);
  if (s->topk < 1) return fail(DSA_ERR_SHAPE, "topk %d < 1", s->topk);
  if (s->flags & ~(DSA_FORCE_SINK | DSA_FORCE_DIAG)) return fail(DSA_ERR_SHAPE, "unknown flags 0x%x", s->flags);
  if ((int64_t)s->batch * s->seq_len * s->n_q_heads >= (1ll << 31))
    return fail(DSA_ERR_UNSUPPORTED, "problem too large for one launch");
  return DSA_OK;
}

int index_kmax(const dsa_index_shape* s) {
  const int N = s->seq_len;
  if (N == 0) return 0;
  int nf = 0;
  if (s->flags & DSA_FORCE_SINK) nf++;
  if ((s->flags & DSA_FORCE_DIAG) && !((s->flags & DSA_FORCE_SINK) && N == 1)) nf++;
  return std::min(N, std::max(s->topk, nf));
}

dsa::TopkParams token_params(const dsa_index_shape* s) {
  return dsa::TopkParams{s->topk,
                         0,
                         1,
                         s->flags,
                         (s->flags & DSA_FORCE_SINK) ? 1 : 0,
                         (s->flags & DSA_FORCE_DIAG) ? 1 : 0,
                         DSA_SELECT_TOPK,
                         0.f,
                         0,
                         0,
                         0};
}

}  // namespace

extern "C" {

const char* dsa_status_str(int status) {
  switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "null pointer";
    case DSA_ERR_SHAPE: return "invalid shape";
    case DSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_err; }

int dsa_prefill_kmax(const dsa_shape* s, int32_t* kmax) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!kmax) return fail(DSA_ERR_NULL, "kmax is NULL");
  *kmax = prefill_kmax(s);
  g_err[0] = 0;
  return DSA_OK;
}

int32_t dsa_kmax(const dsa_shape* s) {
  int rc = check_shape(s);
  if (rc) return rc;
  g_err[0] = 0;
  return s->seq_len > 0 ? row_budget(s, (int)n_blocks(s)) : 0;
}

int dsa_decode_kmax(const dsa_shape* s, int32_t* kmax) {
  int rc = check_decode(s);
  if (rc) return rc;
  if (!kmax) return fail(DSA_ERR_NULL, "kmax is NULL");
  *kmax = s->seq_len > 0 ? row_budget(s, (int)n_blocks(s)) : 0;
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_block_means(const dsa_shape* s, int32_t n_heads, const void* x, float* xbar, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (n_heads < 1) return fail(DSA_ERR_SHAPE, "n_heads %d < 1", n_heads);
  if (empty_prefill(s)) return DSA_OK;
  if (!x || !xbar) return fail(DSA_ERR_NULL, "x or xbar is NULL");
  hipError_t e = dsa::launch_block_means(static_cast<const uint16_t*>(x), xbar, (int64_t)s->batch * n_heads,
                                         s->seq_len, s->head_dim, s->block, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "block_means launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_kv_block_means(const dsa_shape* s, const void* k_cache, float* kbar, void* stream) {
  int rc = check_decode(s);
  if (rc) return rc;
  return dsa_block_means(s, s->n_kv_heads, k_cache, kbar, stream);
}

int dsa_block_scores_from_means(const dsa_shape* s, const float* qbar, const float* kbar, float* scores,
                                void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (empty_prefill(s)) return DSA_OK;
  if (!qbar || !kbar || !scores) return fail(DSA_ERR_NULL, "qbar, kbar or scores is NULL");
  hipError_t e = dsa::launch_block_scores(qbar, kbar, scores, s->batch, s->n_q_heads, s->n_kv_heads, (int)n_blocks(s),
                                          s->head_dim, 1.0f / sqrtf((float)s->head_dim),
                                          static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "block_scores launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_block_scores(const dsa_shape* s, const void* q, const void* k, float* scores, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (empty_prefill(s)) return DSA_OK;
  if (!q || !k || !scores) return fail(DSA_ERR_NULL, "q, k or scores is NULL");
  hipError_t e = dsa::launch_pooled_scores(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), scores,
                                           s->batch, s->n_q_heads, s->n_kv_heads, s->seq_len, s->head_dim, s->block,
                                           1.0f / sqrtf((float)s->head_dim), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pooled block_scores launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_select_topk(const dsa_shape* s, const float* scores, int32_t* idx, int32_t* cnt, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (empty_prefill(s)) return DSA_OK;
  if (!scores || !idx || !cnt) return fail(DSA_ERR_NULL, "scores, idx or cnt is NULL");
  const int nB = (int)n_blocks(s);
  hipError_t e = dsa::launch_select_topk(scores, idx, cnt, (int64_t)s->batch * s->n_kv_heads * nB, nB, nB, true,
                                         topk_params(s), prefill_kmax(s), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "select_topk launch");
  g_err[0] = 0;
  return DSA_OK;
}

static int check_paged(const dsa_shape* s, int32_t n_pages, int32_t max_blocks) {
  int rc = check_decode(s);
  if (rc) return rc;
  if (n_pages < 1) return fail(DSA_ERR_SHAPE, "n_pages %d < 1", n_pages);
  if (max_blocks != n_blocks(s))
    return fail(DSA_ERR_SHAPE, "max_blocks %d != ceil(seq_len %d / block %d)", max_blocks, s->seq_len, s->block);
  if ((int64_t)n_pages * s->n_kv_heads * s->block * s->head_dim >= (1ll << 40))
    return fail(DSA_ERR_UNSUPPORTED, "page pool too large");
  return DSA_OK;
}

int dsa_paged_decode(const dsa_shape* s, const void* q, const void* k_pool, const void* v_pool,
                     const float* kbar_pool, int32_t n_pages, const int32_t* block_table, int32_t max_blocks,
                     const int32_t* lengths, void* o, float* lse, int32_t* idx, int32_t* cnt, void* stream) {
  int rc = check_paged(s, n_pages, max_blocks);
  if (rc) return rc;
  if (s->batch == 0) return DSA_OK;
  if (!q || !k_pool || !v_pool || !kbar_pool || !block_table || !lengths || !o || !idx)
    return fail(DSA_ERR_NULL, "q, k_pool, v_pool, kbar_pool, block_table, lengths, o or idx is NULL");
  dsa::PagedArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kp = static_cast<const uint16_t*>(k_pool);
  a.vp = static_cast<const uint16_t*>(v_pool);
  a.kbar = kbar_pool;
  a.table = block_table;
  a.lengths = lengths;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.idx = idx;
  a.cnt = cnt;
  a.S = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.max_blocks = max_blocks;
  a.n_pages = n_pages;
  a.kmax = row_budget(s, (int)n_blocks(s));
  a.scale = (float)(1.0 / sqrt((double)s->head_dim));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)s->head_dim));
  hipError_t e = dsa::launch_paged_decode(a, s->head_dim, s->block, topk_params(s), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "paged decode launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_paged_decode_fp8(const dsa_shape* s, const void* q, const uint8_t* k8, const uint8_t* v8, const float* k_scale,
                         const float* v_scale, const float* kbar_pool, int32_t n_pages, const int32_t* block_table,
                         int32_t max_blocks, const int32_t* lengths, void* o, float* lse, int32_t* idx, int32_t* cnt,
                         void* stream) {
  int rc = check_paged(s, n_pages, max_blocks);
  if (rc) return rc;
  if (s->batch == 0) return DSA_OK;
  if (!q || !k8 || !v8 || !k_scale || !v_scale || !kbar_pool || !block_table || !lengths || !o || !idx)
    return fail(DSA_ERR_NULL, "q, k8, v8, k_scale, v_scale, kbar_pool, block_table, lengths, o or idx is NULL");
  dsa::PagedArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k8 = k8;
  a.v8 = v8;
  a.ksc = k_scale;
  a.vsc = v_scale;
  a.kbar = kbar_pool;
  a.table = block_table;
  a.lengths = lengths;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.idx = idx;
  a.cnt = cnt;
  a.S = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.max_blocks = max_blocks;
  a.n_pages = n_pages;
  a.kmax = row_budget(s, (int)n_blocks(s));
  a.scale = (float)(1.0 / sqrt((double)s->head_dim));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)s->head_dim));
  hipError_t e = dsa::launch_paged_decode(a, s->head_dim, s->block, topk_params(s), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 paged decode launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_paged_quantize_fp8(const dsa_shape* s, const void* k_pool, const void* v_pool, int32_t n_pages, uint8_t* k8,
                           uint8_t* v8, float* k_scale, float* v_scale, void* stream) {
  int rc = check_decode(s);
  if (rc) return rc;
  if (n_pages < 1) return fail(DSA_ERR_SHAPE, "n_pages %d < 1", n_pages);
  if (!k_pool || !v_pool || !k8 || !v8 || !k_scale || !v_scale)
    return fail(DSA_ERR_NULL, "k_pool, v_pool, k8, v8, k_scale or v_scale is NULL");
  hipError_t e = dsa::launch_paged_quantize(static_cast<const uint16_t*>(k_pool), static_cast<const uint16_t*>(v_pool),
                                            k8, v8, k_scale, v_scale, n_pages, s->n_kv_heads, s->head_dim, s->block,
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 quantize launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_paged_kv_append_fp8(const dsa_shape* s, const void* k_new, const void* v_new, const int32_t* block_table,
                            int32_t max_blocks, int32_t* lengths, uint8_t* k8, uint8_t* v8, float* k_scale,
                            float* v_scale, float* kbar_pool, int32_t n_pages, void* stream) {
  int rc = check_paged(s, n_pages, max_blocks);
  if (rc) return rc;
  if (s->batch == 0) return DSA_OK;
  if (!k_new || !v_new || !block_table || !lengths || !k8 || !v8 || !k_scale || !v_scale || !kbar_pool)
    return fail(DSA_ERR_NULL, "k_new, v_new, block_table, lengths, k8, v8, k_scale, v_scale or kbar_pool is NULL");
  hipError_t e = dsa::launch_kv_append_fp8(static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                                           block_table, lengths, k8, v8, k_scale, v_scale, kbar_pool, s->batch,
                                           s->n_kv_heads, s->head_dim, s->block, max_blocks, n_pages,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 kv append launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_paged_kv_block_means_fp8(const dsa_shape* s, const uint8_t* k8, const float* k_scale, const int32_t* block_table,
                                 int32_t max_blocks, const int32_t* lengths, float* kbar_pool, int32_t n_pages,
                                 void* stream) {
  int rc = check_paged(s, n_pages, max_blocks);
  if (rc) return rc;
  if (s->batch == 0) return DSA_OK;
  if (!k8 || !k_scale || !block_table || !lengths || !kbar_pool)
    return fail(DSA_ERR_NULL, "k8, k_scale, block_table, lengths or kbar_pool is NULL");
  hipError_t e = dsa::launch_paged_means_fp8(k8, k_scale, block_table, lengths, kbar_pool, s->batch, s->n_kv_heads,
                                             s->head_dim, s->block, max_blocks, n_pages,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 paged block means launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_paged_kv_append(const dsa_shape* s, const void* k_new, const void* v_new, const int32_t* block_table,
                        int32_t max_blocks, int32_t* lengths, void* k_pool, void* v_pool, float* kbar_pool,
                        int32_t n_pages, void* stream) {
  int rc = check_paged(s, n_pages, max_blocks);
  if (rc) return rc;
  if (s->batch == 0) return DSA_OK;
  if (!k_new || !v_new || !block_table || !lengths || !k_pool || !v_pool || !kbar_pool)
    return fail(DSA_ERR_NULL, "k_new, v_new, block_table, lengths, k_pool, v_pool or kbar_pool is NULL");
  hipError_t e = dsa::launch_kv_append(static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                                       block_table, lengths, static_cast<uint16_t*>(k_pool),
                                       static_cast<uint16_t*>(v_pool), kbar_pool, s->batch, s->n_kv_heads,
                                       s->head_dim, s->block, max_blocks, n_pages, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv append launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_paged_kv_block_means(const dsa_shape* s, const void* k_pool, const int32_t* block_table, int32_t max_blocks,
                             const int32_t* lengths, float* kbar_pool, int32_t n_pages, void* stream) {
  int rc = check_paged(s, n_pages, max_blocks);
  if (rc) return rc;
  if (s->batch == 0) return DSA_OK;
  if (!k_pool || !block_table || !lengths || !kbar_pool)
    return fail(DSA_ERR_NULL, "k_pool, block_table, lengths or kbar_pool is NULL");
  hipError_t e = dsa::launch_paged_means(static_cast<const uint16_t*>(k_pool), block_table, lengths, kbar_pool,
                                         s->batch, s->n_kv_heads, s->head_dim, s->block, max_blocks, n_pages,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "paged block means launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_index_kmax(const dsa_index_shape* s, int32_t* kmax) {
  int rc = check_index(s);
  if (rc) return rc;
  if (!kmax) return fail(DSA_ERR_NULL, "kmax is NULL");
  *kmax = index_kmax(s);
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_index_scores(const dsa_index_shape* s, const void* qi, const void* ki, const float* wi, float* scores,
                     void* stream) {
  int rc = check_index(s);
  if (rc) return rc;
  if (s->batch == 0 || s->seq_len == 0) return DSA_OK;
  if (!qi || !ki || !wi || !scores) return fail(DSA_ERR_NULL, "qi, ki, wi or scores is NULL");
  hipError_t e = dsa::launch_index_scores(static_cast<const uint16_t*>(qi), static_cast<const uint16_t*>(ki), wi,
                                          scores, s->batch, s->seq_len, s->index_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "index_scores launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_select_tokens(const dsa_index_shape* s, const float* scores, int32_t* idx, int32_t* cnt, void* stream) {
  int rc = check_index(s);
  if (rc) return rc;
  if (s->batch == 0 || s->seq_len == 0) return DSA_OK;
  if (!scores || !idx || !cnt) return fail(DSA_ERR_NULL, "scores, idx or cnt is NULL");
  const int N = s->seq_len;
  if (N > DSA_MAX_TOKENS) return fail(DSA_ERR_UNSUPPORTED, "seq_len %d > %d tokens", N, DSA_MAX_TOKENS);
  hipError_t e = dsa::launch_select_tokens(scores, idx, cnt, (int64_t)s->batch * N, N, token_params(s), index_kmax(s),
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "select_tokens launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_token_attn_fwd(const dsa_index_shape* s, const void* q, const void* k, const void* v, const int32_t* idx,
                       const int32_t* cnt, void* o, float* lse, void* stream) {
  int rc = check_index(s);
  if (rc) return rc;
  if (s->batch == 0 || s->seq_len == 0) return DSA_OK;
  if (!q || !k || !v || !idx || !cnt || !o) return fail(DSA_ERR_NULL, "q, k, v, idx, cnt or o is NULL");
  dsa::TokenAttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.idx = idx;
  a.cnt = cnt;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.N = s->seq_len;
  a.kmax = index_kmax(s);
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)s->head_dim));
  hipError_t e = dsa::launch_token_attn(a, s->head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "token_attn launch");
  g_err[0] = 0;
  return DSA_OK;
}

// the fused selection takes rows of up to INDEX_TOPK_MAX_KEEP kept tokens;
// longer rows go through the scores array
bool index_fused(const dsa_index_shape* s) { return index_kmax(s) <= dsa::INDEX_TOPK_MAX_KEEP; }

size_t dsa_index_workspace_bytes(const dsa_index_shape* s) {
  if (check_index(s)) return 0;
  if (index_fused(s)) return align256(dsa::plan_index_topk(s->batch, s->seq_len, index_kmax(s)).ws_bytes);
  return align256((size_t)s->batch * s->seq_len * s->seq_len * 4);
}

int dsa_index_topk(const dsa_index_shape* s, const void* qi, const void* ki, const float* wi, int32_t* idx,
                   int32_t* cnt, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_index(s);
  if (rc) return rc;
  if (s->batch == 0 || s->seq_len == 0) return DSA_OK;
  if (!qi || !ki || !wi || !idx || !cnt) return fail(DSA_ERR_NULL, "qi, ki, wi, idx or cnt is NULL");
  const int kmax = index_kmax(s);
  if (!index_fused(s))
    return fail(DSA_ERR_UNSUPPORTED, "%d kept tokens per row > %d", kmax, dsa::INDEX_TOPK_MAX_KEEP);
  const size_t need = align256(dsa::plan_index_topk(s->batch, s->seq_len, kmax).ws_bytes);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace %zu bytes at %p, need %zu", ws_bytes, ws, need);
  hipError_t e = dsa::launch_index_topk(static_cast<const uint16_t*>(qi), static_cast<const uint16_t*>(ki), wi, idx,
                                        cnt, ws, s->batch, s->seq_len, s->index_dim, token_params(s), kmax,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "index_topk launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_index_prefill(const dsa_index_shape* s, const void* qi, const void* ki, const float* wi, const void* q,
                      const void* k, const void* v, void* o, float* lse, int32_t* idx, int32_t* cnt, void* ws,
                      size_t ws_bytes, void* stream) {
  int rc = check_index(s);
  if (rc) return rc;
  if (s->batch == 0 || s->seq_len == 0) return DSA_OK;
  if (!qi || !ki || !wi || !q || !k || !v || !o || !idx || !cnt)
    return fail(DSA_ERR_NULL, "qi, ki, wi, q, k, v, o, idx or cnt is NULL");
  if (index_fused(s)) {
    rc = dsa_index_topk(s, qi, ki, wi, idx, cnt, ws, ws_bytes, stream);
    if (rc) return rc;
    return dsa_token_attn_fwd(s, q, k, v, idx, cnt, o, lse, stream);
  }
  if (s->seq_len > DSA_MAX_TOKENS)
    return fail(DSA_ERR_UNSUPPORTED, "seq_len %d > %d tokens with %d kept per row", s->seq_len, DSA_MAX_TOKENS,
                index_kmax(s));
  const size_t need = dsa_index_workspace_bytes(s);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace %zu bytes at %p, need %zu", ws_bytes, ws, need);
  float* scores = static_cast<float*>(ws);
  rc = dsa_index_scores(s, qi, ki, wi, scores, stream);
  if (rc) return rc;
  rc = dsa_select_tokens(s, scores, idx, cnt, stream);
  if (rc) return rc;
  return dsa_token_attn_fwd(s, q, k, v, idx, cnt, o, lse, stream);
}

int dsa_indices_to_bitmap(const int32_t* idx, const int32_t* cnt, int64_t n_rows, int32_t kmax, int32_t n_cols,
                          uint32_t* bitmap, void* stream) {
  if (n_rows < 0 || n_rows >= (1ll << 31)) return fail(DSA_ERR_SHAPE, "n_rows %lld out of range", (long long)n_rows);
  if (kmax < 1) return fail(DSA_ERR_SHAPE, "kmax %d < 1", kmax);
  if (n_cols < 1 || n_cols > DSA_MAX_BLOCKS)
    return fail(DSA_ERR_SHAPE, "n_cols %d not in [1, %d]", n_cols, DSA_MAX_BLOCKS);
  if (n_rows == 0) {
    g_err[0] = 0;
    return DSA_OK;
  }
  if (!idx || !bitmap) return fail(DSA_ERR_NULL, "idx or bitmap is NULL");
  hipError_t e = dsa::launch_bitmap(idx, cnt, bitmap, n_rows, kmax, n_cols, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bitmap launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_sparse_attn_fwd(const dsa_shape* s, const void* q, const void* k, const void* v, const int32_t* idx,
                        const int32_t* cnt, void* o, float* lse, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (empty_prefill(s)) return DSA_OK;
  if (!q || !k || !v || !idx || !cnt || !o) return fail(DSA_ERR_NULL, "q, k, v, idx, cnt or o is NULL");
  dsa::AttnArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.idx = idx;
  a.cnt = cnt;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.N = s->seq_len;
  a.nB = (int)n_blocks(s);
  a.kmax = prefill_kmax(s);
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)s->head_dim));
  hipError_t e = dsa::launch_sparse_attn_fwd(a, s->head_dim, s->block, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sparse_attn_fwd launch");
  g_err[0] = 0;
  return DSA_OK;
}

size_t dsa_attn_bwd_workspace_bytes(const dsa_shape* s) {
  if (check_shape(s)) return 0;
  const size_t nB = (size_t)n_blocks(s), B = (size_t)s->batch, N = (size_t)s->seq_len;
  return align256(B * s->n_q_heads * nB * 2 * (size_t)s->block * 4) + align256(B * s->n_kv_heads * nB * 4) +
         align256(B * s->n_kv_heads * nB * nB * 4);
}

int dsa_sparse_attn_bwd(const dsa_shape* s, const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, const int32_t* idx, const int32_t* cnt, void* dq,
                        void* dk, void* dv, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (empty_prefill(s)) return DSA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !idx || !cnt || !dq || !dk || !dv)
    return fail(DSA_ERR_NULL, "q, k, v, o, lse, dout, idx, cnt, dq, dk or dv is NULL");
  const size_t need = dsa_attn_bwd_workspace_bytes(s);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace %zu bytes at %p, need %zu", ws_bytes, ws, need);
  const size_t nB = (size_t)n_blocks(s), B = (size_t)s->batch, N = (size_t)s->seq_len;
  char* p = static_cast<char*>(ws);
  float* rowstat = reinterpret_cast<float*>(p);
  p += align256(B * s->n_q_heads * nB * 2 * (size_t)s->block * 4);
  int32_t* inv_cnt = reinterpret_cast<int32_t*>(p);
  p += align256(B * s->n_kv_heads * nB * 4);
  int32_t* inv_idx = reinterpret_cast<int32_t*>(p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = dsa::launch_bwd_prep(static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dout), lse, rowstat,
                                      (int64_t)B * s->n_q_heads, (int)N, s->head_dim, s->block, (int)nB, st);
  if (e != hipSuccess) return hip_fail(e, "bwd_prep launch");
  e = dsa::launch_bwd_invert(idx, cnt, inv_cnt, inv_idx, (int64_t)B * s->n_kv_heads, (int)nB, prefill_kmax(s), st);
  if (e != hipSuccess) return hip_fail(e, "bwd_invert launch");
  dsa::BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.dout = static_cast<const uint16_t*>(dout);
  a.rowstat = rowstat;
  a.idx = idx;
  a.cnt = cnt;
  a.inv_cnt = inv_cnt;
  a.inv_idx = inv_idx;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.B = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.N = s->seq_len;
  a.nB = (int)nB;
  a.kmax = prefill_kmax(s);
  a.scale = (float)(1.0 / sqrt((double)s->head_dim));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)s->head_dim));
  e = dsa::launch_sparse_attn_bwd(a, s->head_dim, s->block, st);
  if (e != hipSuccess) return hip_fail(e, "sparse_attn_bwd launch");
  g_err[0] = 0;
  return DSA_OK;
}

size_t dsa_prefill_workspace_bytes(const dsa_shape* s) {
  if (check_shape(s)) return 0;
  const size_t nB = (size_t)n_blocks(s), d = (size_t)s->head_dim, B = (size_t)s->batch;
  return align256(B * s->n_q_heads * nB * d * 4) + align256(B * s->n_kv_heads * nB * d * 4) +
         align256(B * s->n_kv_heads * nB * nB * 4);
}

int dsa_prefill(const dsa_shape* s, const void* q, const void* k, const void* v, void* o, float* lse, int32_t* idx,
                int32_t* cnt, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (empty_prefill(s)) return DSA_OK;
  if (!q || !k || !v || !o || !idx || !cnt) return fail(DSA_ERR_NULL, "q, k, v, o, idx or cnt is NULL");
  const size_t need = dsa_prefill_workspace_bytes(s);
  if (!ws || ws_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace %zu bytes at %p, need %zu", ws_bytes, ws, need);
  const size_t nB = (size_t)n_blocks(s), d = (size_t)s->head_dim, B = (size_t)s->batch;
  char* p = static_cast<char*>(ws);
  float* qbar = reinterpret_cast<float*>(p);
  p += align256(B * s->n_q_heads * nB * d * 4);
  float* kbar = reinterpret_cast<float*>(p);
  p += align256(B * s->n_kv_heads * nB * d * 4);
  float* scores = reinterpret_cast<float*>(p);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = dsa::launch_block_means2(static_cast<const uint16_t*>(q), qbar, (int64_t)B * s->n_q_heads,
                                          static_cast<const uint16_t*>(k), kbar, (int64_t)B * s->n_kv_heads,
                                          s->seq_len, s->head_dim, s->block, st);
  if (e != hipSuccess) return hip_fail(e, "block_means(q, k) launch");
  rc = dsa_block_scores_from_means(s, qbar, kbar, scores, stream);
  if (rc) return rc;
  rc = dsa_select_topk(s, scores, idx, cnt, stream);
  if (rc) return rc;
  return dsa_sparse_attn_fwd(s, q, k, v, idx, cnt, o, lse, stream);
}

size_t dsa_decode_workspace_bytes(const dsa_shape* s) {
  if (check_decode(s)) return 0;
  const size_t nB = (size_t)n_blocks(s), d = (size_t)s->head_dim;
  const size_t units = (size_t)s->batch * s->n_kv_heads;
  if ((int64_t)units >= dsa::DEC_FUSED_MIN_UNITS) return 0;  // one launch, no partials
  const int kmax = s->seq_len > 0 ? row_budget(s, (int)nB) : 0;
  const size_t G = (size_t)(s->n_q_heads / s->n_kv_heads);
  const size_t nsplit = (size_t)dsa::decode_splits(s->batch, s->n_kv_heads, kmax);
  (void)nB;
  return align256(units * nsplit * G * (d + 2) * 4);
}

static int decode_impl(const dsa_shape* s, const void* q, const void* k_cache, const void* v_cache, const float* kbar,
                       void* o, float* lse, int32_t* idx, float* partial, void* stream) {
  const int nB = (int)n_blocks(s);
  const int kmax = row_budget(s, nB);
  dsa::DecodeArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(k_cache);
  a.vc = static_cast<const uint16_t*>(v_cache);
  a.kbar = kbar;
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.idx = idx;
  a.S = s->batch;
  a.Hq = s->n_q_heads;
  a.Hkv = s->n_kv_heads;
  a.L = s->seq_len;
  a.nB = nB;
  a.kmax = kmax;
  a.nsplit = dsa::decode_splits(s->batch, s->n_kv_heads, kmax);
  a.block = s->block;
  a.scale = 1.0f / sqrtf((float)s->head_dim);
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)s->head_dim));
  a.partial = partial;
  hipError_t e = dsa::launch_decode(a, s->head_dim, topk_params(s), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_decode(const dsa_shape* s, const void* q, const void* k_cache, const void* v_cache, const float* kbar,
               void* o, float* lse, int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_decode(s);
  if (rc) return rc;
  if (s->batch == 0) return DSA_OK;
  if (!q || !k_cache || !v_cache || !kbar || !o || !idx)
    return fail(DSA_ERR_NULL, "q, k_cache, v_cache, kbar, o or idx is NULL");
  const size_t need = dsa_decode_workspace_bytes(s);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace %zu bytes at %p, need %zu", ws_bytes, ws, need);
  return decode_impl(s, q, k_cache, v_cache, kbar, o, lse, idx, static_cast<float*>(ws), stream);
}

int dsa_decode_noalloc(const dsa_shape* s, const void* q, const void* k_cache, const void* v_cache, const float* kbar,
                       void* o, float* lse, int32_t* idx, void* stream) {
  int rc = check_decode(s);
  if (rc) return rc;
  if (s->batch == 0) return DSA_OK;
  if (!q || !k_cache || !v_cache || !kbar || !o || !idx)
    return fail(DSA_ERR_NULL, "q, k_cache, v_cache, kbar, o or idx is NULL");
  const size_t need = dsa_decode_workspace_bytes(s);
  if (need > DSA_DECODE_NOALLOC_MAX_BYTES)
    return fail(DSA_ERR_UNSUPPORTED, "decode needs %zu bytes of scratch, more than the %zu the library holds", need,
                (size_t)DSA_DECODE_NOALLOC_MAX_BYTES);
  void* scratch = nullptr;
  hipError_t e = dsa::decode_noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "decode scratch lookup");
  return decode_impl(s, q, k_cache, v_cache, kbar, o, lse, idx, static_cast<float*>(scratch), stream);
}

int dsa_check_block_selection(const dsa_shape* s, int32_t layout, const int32_t* idx, const int32_t* cnt,
                              const int32_t* lengths, int64_t* report, void* stream) {
  if (layout != DSA_LAYOUT_PREFILL && layout != DSA_LAYOUT_DECODE && layout != DSA_LAYOUT_PAGED)
    return fail(DSA_ERR_SHAPE, "unknown layout %d", layout);
  int rc = layout == DSA_LAYOUT_PREFILL ? check_shape(s) : check_decode(s);
  if (rc) return rc;
  if (!report) return fail(DSA_ERR_NULL, "report is NULL");
  const int nB = (int)n_blocks(s);
  dsa::CheckArgs a{};
  a.report = reinterpret_cast<unsigned long long*>(report);
  a.layout = layout;
  if (layout == DSA_LAYOUT_PREFILL) {
    a.n_rows = (int64_t)s->batch * s->n_kv_heads * nB;
    a.kmax = prefill_kmax(s);
    a.period = nB;
  } else {
    a.n_rows = (int64_t)s->batch * s->n_kv_heads;
    a.kmax = s->seq_len > 0 ? row_budget(s, nB) : 0;
    a.period = nB;
    a.per_seq = s->n_kv_heads;
    a.block = s->block;
    a.capacity = s->seq_len;
  }
  if (a.n_rows > 0 && a.kmax > 0) {
    if (!idx) return fail(DSA_ERR_NULL, "idx is NULL");
    if (layout == DSA_LAYOUT_PREFILL && !cnt) return fail(DSA_ERR_NULL, "cnt is NULL (a prefill selection has one)");
    if (layout == DSA_LAYOUT_PAGED && !lengths) return fail(DSA_ERR_NULL, "lengths is NULL");
  } else {
    a.n_rows = 0;  // nothing listed: the report is cleared and ROWS stays 0
  }
  a.idx = idx;
  a.cnt = cnt;
  a.lengths = lengths;
  const dsa::TopkParams p = topk_params(s);
  a.sel_mode = p.mode;
  a.topk = p.topk;
  a.topk_num = p.num;
  a.topk_den = p.den;
  a.anchors = p.anchors;
  a.window = p.window;
  a.cand_cap = p.cand_cap;
  a.k_min = p.k_min;
  a.k_max = p.k_max;
  hipError_t e = dsa::launch_check(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "selection check launch");
  g_err[0] = 0;
  return DSA_OK;
}

int dsa_check_token_selection(const dsa_index_shape* s, const int32_t* idx, const int32_t* cnt, int64_t* report,
                              void* stream) {
  int rc = check_index(s);
  if (rc) return rc;
  if (!report) return fail(DSA_ERR_NULL, "report is NULL");
  dsa::CheckArgs a{};
  a.report = reinterpret_cast<unsigned long long*>(report);
  a.layout = DSA_LAYOUT_PREFILL;  // the row of token t sees t + 1 positions
  a.n_rows = (int64_t)s->batch * s->seq_len;
  a.kmax = index_kmax(s);
  a.period = s->seq_len;
  if (a.n_rows > 0 && !idx) return fail(DSA_ERR_NULL, "idx is NULL");
  a.idx = idx;
  a.cnt = cnt;
  const dsa::TopkParams p = token_params(s);
  a.sel_mode = p.mode;
  a.topk = p.topk;
  a.topk_num = p.num;
  a.topk_den = p.den;
  a.anchors = p.anchors;
  a.window = p.window;
  hipError_t e = dsa::launch_check(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "selection check launch");
  g_err[0] = 0;
  return DSA_OK;
}

}  // extern "C"
