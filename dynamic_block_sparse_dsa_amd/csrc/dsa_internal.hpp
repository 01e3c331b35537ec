// Internal declarations shared by the libdsa HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

// ---------------------------------------------------------------- vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 <-> fp32.  bf16 is the top half of an fp32, so widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Order-preserving map of a finite fp32 onto uint32 (larger float -> larger
// key).  -0.0 is folded onto +0.0 first so equal values get equal keys.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- XCD-aware ids
// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X (id w
// goes to XCD w % 8).  This bijection gives each XCD a contiguous range of
// logical ids, so neighbouring logical work (the query blocks of one head,
// which read the same K/V tiles) shares that XCD's L2.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t w, uint32_t total) {
  const uint32_t xcd = w & 7u, local = w >> 3;
  const uint32_t base = total >> 3, extra = total & 7u;
  return xcd * base + (xcd < extra ? xcd : extra) + local;
}

// ---------------------------------------------------------------- launchers
// Every launcher enqueues on `stream` and returns hipSuccess or the launch
// error.  Sizes are validated by the caller (api.cpp).

// x [n_units, N, d] bf16 -> xbar [n_units, nB, d] fp32 (mean per block)
hipError_t launch_block_means(const uint16_t* x, float* xbar, int64_t n_units, int N, int d, int block,
                              hipStream_t stream);
// the means of two [*, N, d] tensors (n0 and n1 units) in one launch
hipError_t launch_block_means2(const uint16_t* x0, float* xbar0, int64_t n0, const uint16_t* x1, float* xbar1,
                               int64_t n1, int N, int d, int block, hipStream_t stream);

// qbar [B, Hq, nB, d], kbar [B, Hkv, nB, d] -> scores [B, Hkv, nB, nB]
hipError_t launch_block_scores(const float* qbar, const float* kbar, float* scores, int B, int Hq, int Hkv, int nB,
                               int d, float scale, hipStream_t stream);
// q [B, Hq, N, d], k [B, Hkv, N, d] bf16 -> scores [B, Hkv, nB, nB] (the same
// bits as block means followed by launch_block_scores), no workspace
hipError_t launch_pooled_scores(const uint16_t* q, const uint16_t* k, float* scores, int B, int Hq, int Hkv, int N,
                                int d, int block, float scale, hipStream_t stream);

// Selection of one row.  anchors / window are resolved (0 when the matching
// flag is off, >= 1 when on); cand_cap = floor(1 / threshold).
struct TopkParams {
  int topk, num, den;
  uint32_t flags;
  int anchors, window;
  int mode;  // DSA_SELECT_*
  float threshold;
  int k_min, k_max, cand_cap;
};
// rows of `scores` (stride n_cols).  causal: row r sees (r % rows_per_unit) + 1
// blocks; otherwise every row sees n_cols.  idx [n_rows, kmax], cnt [n_rows]
// (cnt may be NULL).
hipError_t launch_select_topk(const float* scores, int32_t* idx, int32_t* cnt, int64_t n_rows, int rows_per_unit,
                              int n_cols, bool causal, TopkParams p, int kmax, hipStream_t stream);

// selection rows [n_rows, kmax] (cnt may be NULL: every row has kmax
// entries) -> bit words [n_rows, ceil(n_cols / 32)]
hipError_t launch_bitmap(const int32_t* idx, const int32_t* cnt, uint32_t* out, int64_t n_rows, int kmax, int n_cols,
                         hipStream_t stream);

// token-level indexer: scores [B, N, N] fp32 (row t written for s <= t)
hipError_t launch_index_scores(const uint16_t* qi, const uint16_t* ki, const float* wi, float* scores, int B, int N,
                               int di, hipStream_t stream);

// token rows of up to 8192 scores: a streaming fast path, then the general
// select for the rows it marks (cnt = -1)
hipError_t launch_select_tokens(const float* scores, int32_t* idx, int32_t* cnt, int64_t n_rows, int N, TopkParams p,
                                int kmax, hipStream_t stream);
hipError_t launch_select_marked(const float* scores, int32_t* idx, int32_t* cnt, int64_t n_rows, int N, TopkParams p,
                                int kmax, hipStream_t stream);

// fused index scores + token selection: token tiles of 16 x chunks of kct
// key tiles of 64; rows whose keys span several chunks keep a list per chunk
// (the best m of it) in the workspace, merged by a second kernel
constexpr int INDEX_TOPK_MAX_KEEP = 128;  // kmax the candidate lists take
constexpr int INDEX_TOPK_MAX_CHUNKS = 2;
// index_merge_kernel holds at most 16 list positions per lane
static_assert(INDEX_TOPK_MAX_CHUNKS * INDEX_TOPK_MAX_KEEP <= 1024, "merge width");
struct IndexTopkArgs {
  const uint16_t* qi;  // [B, N, 16, dI]
  const uint16_t* ki;  // [B, N, dI]
  const float* wi;     // [B, N, 16]
  int32_t* idx;        // [B, N, kmax]
  int32_t* cnt;        // [B, N]
  uint32_t* part_key;  // [B, N, nch, mw] order keys of a chunk's list
  int32_t* part_idx;   // [B, N, nch, mw] their positions
  int32_t* part_cnt;   // [B, N, nch]
  int N, n_tt, kct, nch, mw, kmax;
  TopkParams p;
};
struct IndexTopkPlan {
  int kct, nch, mw;
  size_t ws_bytes;
};
IndexTopkPlan plan_index_topk(int B, int N, int kmax);
hipError_t launch_index_topk(const uint16_t* qi, const uint16_t* ki, const float* wi, int32_t* idx, int32_t* cnt,
                             void* ws, int B, int N, int di, TopkParams p, int kmax, hipStream_t stream);

struct TokenAttnArgs {
  const uint16_t* q;    // [B, Hq, N, d]
  const uint16_t* k;    // [B, Hkv, N, d]
  const uint16_t* v;
  const int32_t* idx;   // [B, N, kmax] kept tokens per query token
  const int32_t* cnt;   // [B, N]
  uint16_t* o;          // [B, Hq, N, d]
  float* lse;           // [B, Hq, N] or null
  int B, Hq, Hkv, N, kmax;
  float scale_log2;     // log2(e) / sqrt(d)
};
hipError_t launch_token_attn(const TokenAttnArgs& a, int d, hipStream_t stream);

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  const int32_t* cnt;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, N, nB, kmax;
  float scale_log2;  // log2(e) / sqrt(d)
};
hipError_t launch_sparse_attn_fwd(const AttnArgs& a, int d, int block, hipStream_t stream);

struct BwdArgs {
  const uint16_t* q;     // [B, Hq, N, d]
  const uint16_t* k;     // [B, Hkv, N, d]
  const uint16_t* v;
  const uint16_t* dout;  // [B, Hq, N, d]
  const float* rowstat;  // [B, Hq, nB, 2, block]: lse log2(e), then rowsum(dO * O); zeros past N
  const int32_t* idx;    // [B, Hkv, nB, kmax]
  const int32_t* cnt;    // [B, Hkv, nB]
  const int32_t* inv_cnt;  // [B, Hkv, nB]
  const int32_t* inv_idx;  // [B, Hkv, nB, nB]
  uint16_t* dq;          // [B, Hq, N, d]
  uint16_t* dk;          // [B, Hkv, N, d]
  uint16_t* dv;
  int B, Hq, Hkv, N, nB, kmax;
  float scale;       // 1 / sqrt(d)
  float scale_log2;  // log2(e) / sqrt(d)
};
hipError_t launch_bwd_prep(const uint16_t* o, const uint16_t* dout, const float* lse, float* rowstat, int64_t n_heads,
                           int N, int d, int block, int nB, hipStream_t stream);
hipError_t launch_bwd_invert(const int32_t* idx, const int32_t* cnt, int32_t* inv_cnt, int32_t* inv_idx,
                             int64_t n_units, int nB, int kmax, hipStream_t stream);
hipError_t launch_sparse_attn_bwd(const BwdArgs& a, int d, int block, hipStream_t stream);

// paged cache: pools [n_pages, Hkv, block, d], means [n_pages, Hkv, d],
// table [S, max_blocks], lengths [S]
struct PagedArgs {
  const uint16_t* q;        // [S, Hq, d]
  const uint16_t* kp;
  const uint16_t* vp;
  const float* kbar;
  const int32_t* table;
  const int32_t* lengths;
  uint16_t* o;              // [S, Hq, d]
  float* lse;               // [S, Hq] or null
  int32_t* idx;             // [S, Hkv, kmax]
  int32_t* cnt;             // [S, Hkv] or null
  int S, Hq, Hkv, max_blocks, n_pages, kmax;
  float scale, scale_log2;  // 1/sqrt(d), log2(e)/sqrt(d)
  // FP8 pools (E4M3 codes [n_pages, Hkv, block, d]) and their row scales
  // [n_pages, Hkv, block]; used instead of kp / vp when set
  const uint8_t* k8;
  const uint8_t* v8;
  const float* ksc;
  const float* vsc;
};
hipError_t launch_paged_decode(const PagedArgs& a, int d, int block, TopkParams p, hipStream_t stream);
hipError_t launch_kv_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* table, int32_t* lengths,
                            uint16_t* kp, uint16_t* vp, float* kbar, int S, int Hkv, int d, int block, int max_blocks,
                            int n_pages, hipStream_t stream);
hipError_t launch_paged_means(const uint16_t* kp, const int32_t* table, const int32_t* lengths, float* kbar, int S,
                              int Hkv, int d, int block, int max_blocks, int n_pages, hipStream_t stream);
// FP8 pools: quantize bf16 pools (every slot), append, page means
hipError_t launch_paged_quantize(const uint16_t* kp, const uint16_t* vp, uint8_t* k8, uint8_t* v8, float* ksc,
                                 float* vsc, int n_pages, int Hkv, int d, int block, hipStream_t stream);
hipError_t launch_kv_append_fp8(const uint16_t* k_new, const uint16_t* v_new, const int32_t* table, int32_t* lengths,
                                uint8_t* k8, uint8_t* v8, float* ksc, float* vsc, float* kbar, int S, int Hkv, int d,
                                int block, int max_blocks, int n_pages, hipStream_t stream);
hipError_t launch_paged_means_fp8(const uint8_t* k8, const float* ksc, const int32_t* table, const int32_t* lengths,
                                  float* kbar, int S, int Hkv, int d, int block, int max_blocks, int n_pages,
                                  hipStream_t stream);

struct DecodeArgs {
  const uint16_t* q;   // [S, Hq, d]
  const uint16_t* kc;  // [S, Hkv, L, d]
  const uint16_t* vc;
  const float* kbar;   // [S, Hkv, nB, d]
  uint16_t* o;         // [S, Hq, d]
  float* lse;          // [S, Hq] or null
  int32_t* idx;        // [S, Hkv, kmax]
  float* partial;      // workspace [S, Hkv, nsplit, G, d + 2]
  int S, Hq, Hkv, L, nB, kmax, nsplit, block;
  float scale;       // 1 / sqrt(d)
  float scale_log2;  // log2(e) / sqrt(d)
};
hipError_t launch_decode(const DecodeArgs& a, int d, TopkParams p, hipStream_t stream);
// device address, on the current device, of the library-owned scratch of
// DSA_DECODE_NOALLOC_MAX_BYTES (looked up once per device)
hipError_t decode_noalloc_scratch(void** out);

// Decode split path: at most DEC_MAX_SPLITS key splits per (sequence, KV
// head); the split count aims at about DEC_TARGET_WG attention workgroups
// (fewer, longer-lived waves that each walk several chunks beat one chunk per
// wave).  decode_splits: the number a step uses (also sizes its workspace).
constexpr int DEC_MAX_SPLITS = 32;
constexpr int DEC_TARGET_WG = 1024;
int decode_splits(int S, int Hkv, int kmax);
// With at least this many (sequence, KV head) units -- one per CU of an
// MI355X -- a decode step is one launch of the fused one-workgroup-per-unit
// kernel, which fills the chip by itself and needs no workspace.
constexpr int64_t DEC_FUSED_MIN_UNITS = 256;

}  // namespace dsa

namespace dsa {

// ---------------------------------------------------------------- selection validator
// Rows r = 0 .. n_rows-1 of idx [n_rows, kmax]; a row sees `visible` ids:
// PREFILL (r % period) + 1 (rows run over the query block / token fastest),
// DECODE period, PAGED ceil(clamp(lengths[r / per_seq], 0, capacity) / block).
// cnt null: a row's count is the length of its list before the first -1.
struct CheckArgs {
  const int32_t* idx;
  const int32_t* cnt;      // [n_rows] or null
  const int32_t* lengths;  // PAGED: [n_rows / per_seq]
  unsigned long long* report;  // [DSA_CHECK_N]
  int64_t n_rows;
  int kmax, layout, period, per_seq, block, capacity;
  int sel_mode, topk, topk_num, topk_den, anchors, window, cand_cap, k_min, k_max;
};
hipError_t launch_check(const CheckArgs& a, hipStream_t stream);

}  // namespace dsa
