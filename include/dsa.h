/*
 * libdsa -- content-aware dynamic block-sparse causal attention for AMD
 * Instinct MI355X (gfx950).
 *
 * The method (sources are cited by page and section):
 *   - "dynamic sparse attention explainer" (zblog.xzdbk.com/559.html),
 *     section "基于Top-k选择的局部-全局混合": per query keep the k
 *     highest-scoring keys and drop the rest, with global + local anchors;
 *     sections "硬件友好的稀疏计算实现" and "工程实践建议": make that
 *     decision per 64x64 or 128x128 block so the kept work stays dense;
 *     section "动态开销与计算收益的权衡": precompute the index data at
 *     cache time; section "前沿方向": GQA/MQA groups share one KV cache.
 *   - "稀疏注意力 vs Flash Attention v2" (pnsm.cn/news/1249548.html),
 *     section 1: content-aware top-k by query-key similarity, the
 *     sparse_attention pseudo-code (softmax of masked logits / sqrt(d_k),
 *     times V), and FlashAttention-2's tiling with an incremental softmax.
 *   - DeepSeek NSA article (pnsm.cn/news/1939904.html), section 2.2:
 *     routing scores in fp32, the weighted sum in bf16.
 *
 * One prefill call runs four steps:
 *   1. block means of Q and K (fp32)                 dsa_block_means
 *   2. block scores, causal, max over a GQA group     dsa_block_scores (from
 *                                                    Q, K) or
 *                                                    dsa_block_scores_from_means
 *   3. top-k blocks per query block, sink and
 *      diagonal forced                               dsa_select_topk
 *   4. attention over the kept tiles                  dsa_sparse_attn_fwd
 * dsa_prefill chains them; dsa_decode is the single-token variant;
 * dsa_kmax gives the index width both write.
 *
 * Conventions for every call below:
 *   - All tensor pointers are DEVICE pointers, contiguous, row-major.  bf16
 *     tensors are passed as their 16-bit storage (void*).
 *   - Layouts: Q, O [B, Hq, N, d]; K, V [B, Hkv, N, d]; block means
 *     [B, H, nB, d] fp32; scores [B, Hkv, nB, nB] fp32; idx [B, Hkv, nB, kmax]
 *     int32; cnt [B, Hkv, nB] int32; LSE [B, Hq, N] fp32 (natural log).
 *     nB = ceil(N / block); a ragged last block is allowed (its mean is over
 *     the rows it has).  Query head h reads KV head h / (Hq / Hkv).
 *   - Ownership: the caller owns every buffer.  The library allocates no
 *     memory, keeps no state between calls and is re-entrant; scratch space
 *     comes from the caller's workspace (sizes from *_workspace_bytes).
 *   - Errors: every call returns DSA_OK (0) or a negative DSA_ERR_* code.
 *     Argument errors are detected on the host before anything is enqueued;
 *     launch errors are reported from the HIP runtime.  Work is enqueued
 *     asynchronously on `stream` (a hipStream_t; NULL = the null stream) and
 *     no call synchronises, so device faults surface at the caller's next
 *     synchronisation.  dsa_last_error() gives the calling thread's message.
 *   - Inputs are assumed finite.  An empty problem (B == 0 or N == 0 for
 *     prefill, S == 0 for decode) returns DSA_OK and enqueues nothing.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DSA_OK = 0,
  DSA_ERR_NULL = -1,        /* a required pointer is NULL */
  DSA_ERR_SHAPE = -2,       /* sizes are inconsistent (e.g. Hq % Hkv != 0) */
  DSA_ERR_UNSUPPORTED = -3, /* head_dim / block not built, too many blocks */
  DSA_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than required */
  DSA_ERR_HIP = -5          /* the HIP runtime reported an error */
};

/* flags: which blocks every row keeps regardless of score */
#define DSA_FORCE_SINK 1u /* block 0 */
#define DSA_FORCE_DIAG 2u /* the row's own block: the diagonal block in prefill,
                             the last cache block in decode */
/* and how the work is ordered: with DSA_DETERMINISTIC a decode step gives the
 * same bits on every call (dsa_decode's one-launch path, S * Hkv >= 256, and
 * every dsa_paged_decode / dsa_paged_decode_fp8 call then hand the kept
 * chunks to their waves in a fixed order instead of first come first served;
 * every other call gives the same bits on every call regardless) */
#define DSA_DETERMINISTIC 4u

/* select_mode: how a row's budget is set (prefill; decode takes TOPK only) */
#define DSA_SELECT_TOPK 0      /* topk or the fraction below */
#define DSA_SELECT_THRESHOLD 1 /* every candidate whose share of the row's
                                  block softmax is >= threshold */
#define DSA_SELECT_ENTROPY 2   /* ceil(exp(H)) blocks, H the entropy of that
                                  softmax, clamped to [k_min, k_max] */

/* limits of the built kernels */
#define DSA_MAX_BLOCKS 4096 /* nB = ceil(N / block) */

typedef struct dsa_shape {
  int32_t batch;      /* B (prefill) or number of sequences S (decode), >= 0 */
  int32_t n_q_heads;  /* Hq >= 1 */
  int32_t n_kv_heads; /* Hkv >= 1, Hq % Hkv == 0 (Hkv == Hq: one selection per head) */
  int32_t seq_len;    /* prefill: N >= 0; decode: cache length L >= 1 (the new
                         token is at position L - 1 and is already in the cache) */
  int32_t head_dim;   /* d: 64 or 128 */
  int32_t block;      /* b: 64 or 128 */
  int32_t topk;       /* > 0: blocks kept per row, forced ones included;
                         0: use the fraction below */
  int32_t topk_num;   /* topk == 0: keep ceil(topk_num * visible / topk_den)  */
  int32_t topk_den;   /*   blocks (integer arithmetic), num >= 0, den >= 1    */
  uint32_t flags;     /* DSA_FORCE_SINK | DSA_FORCE_DIAG (or a subset),
                         | DSA_DETERMINISTIC */
  /* Selection variants.  All zero: DSA_SELECT_TOPK with a one-block sink and
   * a one-block diagonal.  "dynamic sparse attention explainer", section
   * "基于Top-k选择的局部-全局混合" (global tokens + a local window), DeepSeek
   * NSA article section 2.2 (block-sparsify the fp32 scores with a
   * threshold), explainer sections "模型精度与稀疏度的动态平衡" and
   * "工程实践建议" (set k or the threshold from the attention entropy). */
  int32_t select_mode; /* DSA_SELECT_* */
  int32_t n_anchor;    /* with DSA_FORCE_SINK: blocks 0 .. n_anchor-1 forced
                          (global anchors); 0 means 1 */
  int32_t window;      /* with DSA_FORCE_DIAG: the last `window` visible blocks
                          forced (a local window ending at the row's own
                          block); 0 means 1 */
  float threshold;     /* DSA_SELECT_THRESHOLD: tau in (0, 1] */
  int32_t k_min;       /* DSA_SELECT_ENTROPY: 1 <= k_min <= k_max */
  int32_t k_max;
} dsa_shape;

/* The row's block distribution is p_j = softmax over its visible blocks of
 * the block scores (forced blocks included).  A row that sees `visible`
 * blocks and has F forced blocks keeps the forced blocks plus:
 *   TOPK:       the best min(max(k, F), visible) - F candidates, k = topk or
 *               the fraction above;
 *   THRESHOLD:  every candidate with p_j >= threshold (at most
 *               floor(1 / threshold) of them);
 *   ENTROPY:    the best min(max(clamp(ceil(exp(H)), k_min, k_max), F),
 *               visible) - F candidates, H = -sum p_j ln p_j.
 * Kept blocks are listed ascending; the rest of the row of idx is -1.
 * Ties in score go to the lower block index.  The decisions at a threshold
 * or an integer exp(H) are taken in fp32. */

/* Width of the index array idx (its last dimension) for a prefill or a
 * decode of this shape: the largest per-row budget, min(max(k, F), nB) for
 * top-k (k = topk or the fraction of nB), F + floor(1 / threshold) for
 * THRESHOLD and max(k_max, F) for ENTROPY, each capped at nB (F = forced
 * blocks of a row that sees all nB blocks; a row's budget never shrinks as it
 * sees more blocks, so the last row's is the largest).  The index lives in
 * caller-preallocated contiguous memory of this width ("低成本高性能大模型实现
 * 路径", section 3.1 "内存访问优化": sparse indices in preallocated contiguous
 * blocks).  Host only; reads nothing but *shape.
 * Returns kmax >= 0 (0 when seq_len == 0), or a negative DSA_ERR_* code. */
int32_t dsa_kmax(const dsa_shape* shape);

/* The same width through an out-parameter, with the checks of the prefill
 * (dsa_prefill_kmax) or decode (dsa_decode_kmax) entry points: the decode
 * form also rejects what dsa_decode does not take (select_mode != TOPK, group
 * sizes other than 1, 2, 4, 8).  Returns DSA_OK and writes *kmax. */
int dsa_prefill_kmax(const dsa_shape* shape, int32_t* kmax);
int dsa_decode_kmax(const dsa_shape* shape, int32_t* kmax);

/* Step 1 on its own: block means.  x: [B, n_heads, N, d] bf16 -> xbar:
 * [B, n_heads, nB, d] fp32 (N = shape->seq_len, B = shape->batch): the mean
 * of each block's rows (a ragged last block over its real rows), summed in
 * fp32 in a fixed order.  Used for Q (n_heads = Hq), K (n_heads = Hkv) and
 * a decode key cache (dsa_kv_block_means).  fp32 because the selection is
 * made from these values (DeepSeek NSA article, section 2.2: routing in
 * fp32).  The block statistic itself -- one summary per tile that the
 * per-block decision compares -- follows "dynamic sparse attention
 * explainer", section "硬件友好的稀疏计算实现" (decide per 64x64 or 128x128
 * block).  Errors: NULL x/xbar, n_heads < 1, shape errors.  Async on stream. */
int dsa_block_means(const dsa_shape* shape, int32_t n_heads, const void* x, float* xbar, void* stream);

/* Step 2: block scores from Q and K.  q [B, Hq, N, d], k [B, Hkv, N, d]
 * bf16 (device) -> scores [B, Hkv, nB, nB] fp32 (device, caller-owned):
 *   scores[b, g, i, j] = max over the query heads h of group g of
 *                        (1/sqrt(d)) * <mean(Q_h block i), mean(K_g block j)>
 * for j <= i, and -inf for j > i.  The means are pooled inside the call
 * (no workspace; they are the bits of dsa_block_means) and the result is
 * bit-identical to dsa_block_means + dsa_block_scores_from_means.  Sources:
 * "稀疏注意力 vs Flash Attention v2" section 1 (content-aware sparsity ranks
 * keys by query-key similarity); "dynamic sparse attention explainer",
 * "前沿方向" (a GQA group shares one KV cache, hence one selection: the max
 * over its heads).  Reads Q and K about nB / 256 times over (a strip of
 * block means is pooled per workgroup); dsa_prefill, which has a workspace,
 * pools each block once.  Errors: NULL q/k/scores, shape errors. */
int dsa_block_scores(const dsa_shape* shape, const void* q, const void* k, float* scores, void* stream);

/* Step 2 from precomputed block means: qbar [B, Hq, nB, d], kbar
 * [B, Hkv, nB, d] fp32 (dsa_block_means) -> scores as dsa_block_scores. */
int dsa_block_scores_from_means(const dsa_shape* shape, const float* qbar, const float* kbar, float* scores,
                                void* stream);

/* Step 3: per-row selection from a score matrix [B, Hkv, nB, nB] fp32 (only
 * j <= i is read).  Row i keeps the forced blocks (DSA_FORCE_SINK: block 0
 * or the first n_anchor blocks; DSA_FORCE_DIAG: block i or the last `window`
 * visible blocks) plus the best-scoring other blocks up to its budget (the
 * rules above; exact ties to the lower block index).  Output idx
 * [B, Hkv, nB, dsa_kmax(shape)] int32, ascending, -1 padded; cnt [B, Hkv, nB]
 * int32, the number kept.  Sources: "dynamic sparse attention explainer",
 * "基于Top-k选择的局部-全局混合" (keep each query's k best keys, drop the rest;
 * global + local anchors) and "硬件友好的稀疏计算实现" (per-block decision).
 * Errors: NULL scores/idx/cnt, shape errors. */
int dsa_select_topk(const dsa_shape* shape, const float* scores, int32_t* idx, int32_t* cnt, void* stream);

/* Step 4: causal attention over the listed blocks.  q [B, Hq, N, d], k, v
 * [B, Hkv, N, d] bf16; idx, cnt as dsa_select_topk writes them (entries
 * 0..cnt-1 of a row must be ascending, distinct, in 0..i -- not checked;
 * counts outside [0, kmax] and block ids outside [0, nB) are clamped into
 * range, so such input gives wrong results but no access outside the
 * tensors).
 * Row p of query block i attends to the keys c <= p of its kept blocks:
 *   O[p] = sum_c softmax_c((1/sqrt(d)) q_p . k_c) v_c,  LSE[p] = log sum_c
 *   exp((1/sqrt(d)) q_p . k_c)
 * with bf16 MFMA products, fp32 accumulation and online softmax, P rounded to
 * bf16 for the P V product.  o [B, Hq, N, d] bf16; lse [B, Hq, N] fp32
 * natural log, or NULL to skip it.  Sources: "稀疏注意力 vs Flash Attention
 * v2" section 1 (the sparse_attention definition: logits, apply the pattern,
 * softmax of logits / sqrt(d_k), times V; FlashAttention-2's tiled
 * incremental softmax); "dynamic sparse attention explainer", "硬件友好的稀疏
 * 计算实现" and "工程实践建议" (kept 64x64 / 128x128 blocks stay dense); DeepSeek
 * NSA article section 2.2 (weighted sum in bf16).  Errors: NULL q/k/v/idx/
 * cnt/o, shape errors. */
int dsa_sparse_attn_fwd(const dsa_shape* shape, const void* q, const void* k, const void* v, const int32_t* idx,
                        const int32_t* cnt, void* o, float* lse, void* stream);

/* Workspace for dsa_prefill, in bytes (block means of Q and K + scores,
 * each 256-byte aligned).  0 for an invalid shape.  Host only. */
size_t dsa_prefill_workspace_bytes(const dsa_shape* shape);

/* Steps 1-4 in one call: Q/K/V in, a block size and k (in *shape), output
 * plus the selected block indices out ("稀疏注意力 vs Flash Attention v2"
 * section 1: sparse_attention(query, key, value, pattern); "dynamic sparse
 * attention explainer", "基于Top-k选择的局部-全局混合").  q, k, v, o, lse as
 * dsa_sparse_attn_fwd; idx, cnt as dsa_select_topk.  ws: device workspace
 * of at least dsa_prefill_workspace_bytes(shape) bytes (caller-owned); after
 * the call it holds the Q means, the K means, then the scores.  Errors as
 * the steps, plus DSA_ERR_WORKSPACE. */
int dsa_prefill(const dsa_shape* shape, const void* q, const void* k, const void* v, void* o, float* lse,
                int32_t* idx, int32_t* cnt, void* ws, size_t ws_bytes, void* stream);

/* Cache-time block means of a decode key cache: k_cache [S, Hkv, L, d] bf16
 * -> kbar [S, Hkv, nB, d] fp32 -- the index data built when the cache is
 * written, so a decode step does not re-pool raw keys ("dynamic sparse
 * attention explainer", "动态开销与计算收益的权衡": precompute at cache time).
 * Errors: as dsa_block_means plus the decode shape checks. */
int dsa_kv_block_means(const dsa_shape* shape, const void* k_cache, float* kbar, void* stream);

/* Workspace for dsa_decode, in bytes (split partials; 0 when the step runs
 * as one workgroup per (sequence, KV head), i.e. S * Hkv >= 256). */
size_t dsa_decode_workspace_bytes(const dsa_shape* shape);

/* One decode step for S sequences.  q: [S, Hq, d] bf16 (the new tokens, at
 * cache position L - 1); k_cache, v_cache: [S, Hkv, L, d] bf16; kbar: the
 * dsa_kv_block_means of k_cache.  Per (sequence, KV head) the blocks are
 * scored by max over the group's heads of (1/sqrt(d)) q_h . kbar_j, the
 * sink and the last block are forced (per flags), the best others fill the
 * budget (ties to the lower block), and every key of the kept blocks is
 * attended to (split over the kept blocks, partials merged).
 * o: [S, Hq, d] bf16; lse: [S, Hq] fp32 or NULL; idx: [S, Hkv, dsa_kmax]
 * int32.  ws: at least dsa_decode_workspace_bytes (NULL allowed when that is
 * 0).  Sources: "dynamic sparse
 * attention explainer", "动态开销与计算收益的权衡" (cache-time index data),
 * "前沿方向" (one selection per GQA group), "硬件友好的稀疏计算实现" (whole
 * blocks of the cache).  Errors: NULL pointers, shape errors (decode takes
 * DSA_SELECT_TOPK only; group sizes 1, 2, 4, 8), DSA_ERR_WORKSPACE. */
int dsa_decode(const dsa_shape* shape, const void* q, const void* k_cache, const void* v_cache, const float* kbar,
               void* o, float* lse, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/* Size of the device scratch dsa_decode_noalloc uses on each GPU (bytes). */
#define DSA_DECODE_NOALLOC_MAX_BYTES (8u << 20)

/* dsa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results as dsa_decode, minus the workspace: the split-path
 * partials go to a device array the library owns, DSA_DECODE_NOALLOC_MAX_BYTES
 * per GPU, held from the first call on that GPU until the process ends.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library call).
 * Every shape dsa_decode takes fits; a shape whose dsa_decode_workspace_bytes
 * exceeded the array would get DSA_ERR_UNSUPPORTED.  All calls on one GPU
 * share the array: calls that overlap on one GPU (e.g. on two streams) race,
 * so serialise them.  Nothing in the array needs to start at zero. */
int dsa_decode_noalloc(const dsa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
                       const float* kbar, void* o, float* lse, int32_t* idx, void* stream);

/* ---- Backward of step 4 (gradients through the kept tiles; the selection
 * is a discrete choice and is held fixed).  The chain rule through the
 * attention definition of "稀疏注意力 vs Flash Attention v2" section 1, with P
 * recomputed from the saved LSE (the FlashAttention-2 recompute idea of the
 * same section): D = rowsum(dO * O), P = exp((1/sqrt(d)) q k^T - lse),
 * dS = P * (dO V^T - D), dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d),
 * dV = P^T dO; dK and dV of a KV head sum its group's query heads.  Keys no
 * row kept get zero gradients. */

/* Workspace for dsa_sparse_attn_bwd, in bytes: per query row the LSE in
 * log2 units and D, fp32 [B, Hq, nB, 2, block] (rows past N zero-padded),
 * and the inverted selection (per KV block, the query blocks that kept it)
 * [B, Hkv, nB] + [B, Hkv, nB, nB] int32. */
size_t dsa_attn_bwd_workspace_bytes(const dsa_shape* shape);

/* q, k, v, idx, cnt as given to dsa_sparse_attn_fwd; o and lse (required)
 * as it returned them; dout: dL/dO [B, Hq, N, d] bf16.  Writes dq
 * [B, Hq, N, d], dk and dv [B, Hkv, N, d], bf16 (fp32 accumulation; P and
 * dS are rounded to bf16 as MFMA operands).  Every element of dq, dk, dv is
 * written.  ws: at least dsa_attn_bwd_workspace_bytes. */
int dsa_sparse_attn_bwd(const dsa_shape* shape, const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, const int32_t* idx, const int32_t* cnt, void* dq,
                        void* dk, void* dv, void* ws, size_t ws_bytes, void* stream);

/* ---- Paged decode with a length per sequence ("dynamic sparse attention
 * explainer": "硬件友好的稀疏计算实现" ties the block decision to the KV
 * cache's blocks; "动态开销与计算收益的权衡" builds the index data when the
 * cache is written).  A page holds one block (shape->block tokens) of one
 * sequence for every KV head:
 *   k_pool, v_pool [n_pages, Hkv, block, d] bf16;
 *   kbar_pool [n_pages, Hkv, d] fp32, each page's key mean;
 *   block_table [S, max_blocks] int32, the page of logical block j of s;
 *   lengths [S] int32, the tokens in each sequence's cache (device memory).
 * shape: batch = S, heads, head_dim, block, topk / fraction, flags,
 * n_anchor, window as for dsa_decode (select_mode DSA_SELECT_TOPK), and
 * seq_len = the capacity, with max_blocks == ceil(seq_len / block); idx is
 * [S, Hkv, dsa_decode_kmax(shape)].
 * Sequence s (0 <= lengths[s] <= seq_len) is decoded over its first
 * lengths[s] tokens exactly as dsa_decode with L = lengths[s] (its last block
 * may be partial; its new token is at lengths[s] - 1); cnt [S, Hkv]
 * (nullable) gets the kept counts, idx rows are -1 padded; an empty
 * sequence gives o = 0, lse = -inf, cnt = 0.  The table entries of a
 * sequence's first ceil(lengths[s] / block) blocks must name pages in
 * [0, n_pages) (other entries are never read; out-of-range ones are clamped,
 * never dereferenced).  The same bits on every call with DSA_DETERMINISTIC;
 * without it the merge order of the kept chunks varies (rounding only). */
int dsa_paged_decode(const dsa_shape* shape, const void* q, const void* k_pool, const void* v_pool,
                     const float* kbar_pool, int32_t n_pages, const int32_t* block_table, int32_t max_blocks,
                     const int32_t* lengths, void* o, float* lse, int32_t* idx, int32_t* cnt, void* stream);

/* Append one token per sequence: k_new, v_new [S, Hkv, d] bf16 go to
 * position lengths[s] (page block_table[s][lengths[s] / block], slot
 * lengths[s] % block); that page's key mean is recomputed over its rows 0 ..
 * slot (summed in row order, as dsa_paged_kv_block_means does, so both give
 * the same bits); lengths[s] is then incremented in place.  A sequence
 * already holding seq_len tokens, or whose page is out of range, is left
 * unchanged. */
int dsa_paged_kv_append(const dsa_shape* shape, const void* k_new, const void* v_new, const int32_t* block_table,
                        int32_t max_blocks, int32_t* lengths, void* k_pool, void* v_pool, float* kbar_pool,
                        int32_t n_pages, void* stream);

/* Key means of the pages in use: for every sequence s and logical block
 * j < ceil(lengths[s] / block), kbar_pool[block_table[s][j]] = the mean of
 * that page's rows below lengths[s].  Other pages are not written. */
int dsa_paged_kv_block_means(const dsa_shape* shape, const void* k_pool, const int32_t* block_table,
                             int32_t max_blocks, const int32_t* lengths, float* kbar_pool, int32_t n_pages,
                             void* stream);

/* ---- FP8 paged cache ("dynamic sparse attention explainer", "工程实践建议":
 * combine the sparsity with an FP8/INT4 KV cache to cut bandwidth).  The
 * pools hold E4M3 (OCP) codes k8, v8 [n_pages, Hkv, block, d] uint8 with one
 * fp32 scale per (token, KV head) row, k_scale, v_scale [n_pages, Hkv,
 * block]: scale = amax(|row|) / 448 (1 for an all-zero row) and code = the
 * E4M3 value nearest to fp32(x / scale), ties to even; a row's value is
 * code * scale.  The page means, the selection and the attention use those
 * values (attention: bf16 MFMA on the codes, the K scale applied to each
 * logit and the V scale to each softmax weight, fp32 accumulation).  Same
 * layouts and rules as the bf16 paged calls otherwise. */

/* Quantize whole bf16 pools (every slot of every page) into an FP8 cache. */
int dsa_paged_quantize_fp8(const dsa_shape* shape, const void* k_pool, const void* v_pool, int32_t n_pages,
                           uint8_t* k8, uint8_t* v8, float* k_scale, float* v_scale, void* stream);

/* dsa_paged_decode over an FP8 cache. */
int dsa_paged_decode_fp8(const dsa_shape* shape, const void* q, const uint8_t* k8, const uint8_t* v8,
                         const float* k_scale, const float* v_scale, const float* kbar_pool, int32_t n_pages,
                         const int32_t* block_table, int32_t max_blocks, const int32_t* lengths, void* o, float* lse,
                         int32_t* idx, int32_t* cnt, void* stream);

/* dsa_paged_kv_append into an FP8 cache: k_new, v_new [S, Hkv, d] bf16 are
 * quantized row by row; the page mean is recomputed from the page's
 * dequantized rows in row order (the same bits as
 * dsa_paged_kv_block_means_fp8). */
int dsa_paged_kv_append_fp8(const dsa_shape* shape, const void* k_new, const void* v_new, const int32_t* block_table,
                            int32_t max_blocks, int32_t* lengths, uint8_t* k8, uint8_t* v8, float* k_scale,
                            float* v_scale, float* kbar_pool, int32_t n_pages, void* stream);

/* dsa_paged_kv_block_means over an FP8 cache (means of the dequantized rows). */
int dsa_paged_kv_block_means_fp8(const dsa_shape* shape, const uint8_t* k8, const float* k_scale,
                                 const int32_t* block_table, int32_t max_blocks, const int32_t* lengths,
                                 float* kbar_pool, int32_t n_pages, void* stream);

/* ---- Token-level lightning indexer ("低成本高性能大模型实现路径：从架构创新
 * 到工程优化", yunthe.com/news/806485.html, section 2.1 "轻量化索引器设计":
 * ReLU feature heads, 16 index heads, every query token keeps its top 64
 * key/value tokens; section 2.2: low-precision indexer intermediates).  For
 * query token t and earlier token s (s <= t)
 *     I[t, s] = sum_h wi[t, h] * max(0, qi[t, h] . ki[s])
 * (bf16 inputs, fp32 products and sums).  Each query token keeps the forced
 * tokens (DSA_FORCE_SINK: token 0; DSA_FORCE_DIAG: t itself) plus its best
 * other tokens up to topk in all (ties to the lower position), listed
 * ascending, and every attention head of the token attends over exactly
 * those tokens (softmax of q . k / sqrt(d), times v: bf16 products with
 * fp32 accumulation and an fp32 softmax whose weights are rounded to bf16
 * for the product with v, as in dsa_sparse_attn_fwd).
 * Layouts: qi [B, N, HI, dI] bf16; ki [B, N, dI] bf16; wi [B, N, HI] fp32;
 * scores [B, N, N] fp32 (row t: entries 0..t are written, the rest is not
 * touched); idx [B, N, kmax] int32 (-1 padded); cnt [B, N] int32; q, o
 * [B, Hq, N, d] bf16; k, v [B, Hkv, N, d] bf16; lse [B, Hq, N] fp32
 * (natural log, nullable).  Query head h reads KV head h / (Hq / Hkv). */
#define DSA_INDEX_HEADS 16  /* HI, the only index head count built */
#define DSA_MAX_TOKENS 8192 /* longest sequence dsa_select_tokens takes (rows of the scores array) */
#define DSA_INDEX_TOPK_MAX_KEEP 128 /* longest kept row (kmax) dsa_index_topk takes */

typedef struct dsa_index_shape {
  int32_t batch;         /* B >= 0 */
  int32_t n_q_heads;     /* Hq >= 1 */
  int32_t n_kv_heads;    /* Hkv >= 1, Hq / Hkv in {1, 2, 4, 8} */
  int32_t seq_len;       /* N >= 0 (B * N * Hq < 2^31) */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t n_index_heads; /* HI: DSA_INDEX_HEADS */
  int32_t index_dim;     /* dI: 64 or 128 */
  int32_t topk;          /* tokens kept per query token, forced ones included, >= 1 */
  uint32_t flags;        /* DSA_FORCE_SINK | DSA_FORCE_DIAG (or a subset) */
} dsa_index_shape;

/* Width of the token index array: the largest per-row count,
 * min(N, max(topk, forced)).  Host only. */
int dsa_index_kmax(const dsa_index_shape* shape, int32_t* kmax);

/* Index scores I (above) into scores. */
int dsa_index_scores(const dsa_index_shape* shape, const void* qi, const void* ki, const float* wi, float* scores,
                     void* stream);

/* Per query token, the kept tokens from a scores array as written by
 * dsa_index_scores.  N <= DSA_MAX_TOKENS, else DSA_ERR_UNSUPPORTED. */
int dsa_select_tokens(const dsa_index_shape* shape, const float* scores, int32_t* idx, int32_t* cnt, void* stream);

/* Attention of every head over its token's kept tokens.  idx entries are
 * read for the first cnt of each row and must be positions <= t (repeats
 * count once per occurrence).  A row with cnt = 0 gives O = 0 and LSE = -inf. */
int dsa_token_attn_fwd(const dsa_index_shape* shape, const void* q, const void* k, const void* v, const int32_t* idx,
                       const int32_t* cnt, void* o, float* lse, void* stream);

/* Index scores and token selection in one pass (same definition and result
 * as dsa_index_scores then dsa_select_tokens, without the scores array):
 * each query token keeps its forced tokens and its best other tokens by I,
 * ties to the lower position, written to idx [B, N, kmax] (ascending, -1
 * padded) and cnt [B, N].  Takes kmax <= DSA_INDEX_TOPK_MAX_KEEP (else
 * DSA_ERR_UNSUPPORTED) and any N.  ws: device memory of at least
 * dsa_index_workspace_bytes(shape) bytes (the per-chunk candidate lists of
 * rows longer than one chunk of keys; 0 bytes when N <= 2048, NULL then
 * allowed), caller-owned, contents undefined afterwards; DSA_ERR_WORKSPACE
 * if smaller. */
int dsa_index_topk(const dsa_index_shape* shape, const void* qi, const void* ki, const float* wi, int32_t* idx,
                   int32_t* cnt, void* ws, size_t ws_bytes, void* stream);

/* Workspace of dsa_index_prefill and dsa_index_topk in bytes: the candidate
 * lists of dsa_index_topk when kmax <= DSA_INDEX_TOPK_MAX_KEEP, else the
 * scores array, B * N * N * 4 (those shapes need N <= DSA_MAX_TOKENS). */
size_t dsa_index_workspace_bytes(const dsa_index_shape* shape);

/* Selection (dsa_index_topk, or dsa_index_scores then dsa_select_tokens for
 * kmax > DSA_INDEX_TOPK_MAX_KEEP) then dsa_token_attn_fwd. */
int dsa_index_prefill(const dsa_index_shape* shape, const void* qi, const void* ki, const float* wi, const void* q,
                      const void* k, const void* v, void* o, float* lse, int32_t* idx, int32_t* cnt, void* ws,
                      size_t ws_bytes, void* stream);

/* ---- Selection as a bitmap ("dynamic sparse attention explainer", section
 * "工程实践建议": store the sparse index as a compressed bitmap rather than a
 * full index array).  idx [n_rows, kmax] int32 as written by the selection
 * calls (entries outside [0, n_cols), such as the -1 padding, are skipped);
 * cnt [n_rows] int32, or NULL when every row lists kmax blocks (decode).
 * Writes every word of bitmap [n_rows, ceil(n_cols / 32)] uint32: bit j % 32
 * of word j / 32 is set when block j is listed.  Prefill: n_rows =
 * B * Hkv * nB, kmax = dsa_prefill_kmax, n_cols = nB; decode: n_rows =
 * S * Hkv, kmax = dsa_decode_kmax, n_cols = nB, cnt = NULL.
 * 0 <= n_rows < 2^31, kmax >= 1, 1 <= n_cols <= DSA_MAX_BLOCKS. */
int dsa_indices_to_bitmap(const int32_t* idx, const int32_t* cnt, int64_t n_rows, int32_t kmax, int32_t n_cols,
                          uint32_t* bitmap, void* stream);

/* ---- Selection validator (a debug check for index arrays that come from
 * outside the library; the attention kernels only clamp what they read).
 * Counts, without trapping, every way idx breaks the rules the selection
 * calls above write it by, into report[DSA_CHECK_N] (device memory, int64,
 * overwritten: the call clears it on the stream first, with a kernel):
 *   ROWS     rows examined;
 *   COUNT    rows whose count is outside what the selection rule allows for
 *            the row's visible ids (TOPK: exactly min(max(k, F), visible);
 *            THRESHOLD: F .. F + floor(1 / threshold); ENTROPY: between the
 *            k_min and k_max budgets; F the row's forced count) or above kmax;
 *   RANGE    listed ids outside 0 .. visible - 1 (the causal range);
 *   ORDER    adjacent listed pairs that are not strictly ascending (repeats
 *            included);
 *   FORCED   forced ids (anchors and window of the flags) that are not
 *            listed;
 *   PADDING  entries past the count that are not -1.
 * Every slot but ROWS is 0 for an array that a selection call wrote for the
 * same shape.  The rules are those stated with dsa_shape and
 * dsa_index_shape. */
#define DSA_CHECK_N 6
#define DSA_CHECK_ROWS 0
#define DSA_CHECK_COUNT 1
#define DSA_CHECK_RANGE 2
#define DSA_CHECK_ORDER 3
#define DSA_CHECK_FORCED 4
#define DSA_CHECK_PADDING 5

/* Index array layouts for dsa_check_block_selection.
 *   PREFILL: idx [B, Hkv, nB, dsa_prefill_kmax] and cnt [B, Hkv, nB] as
 *            dsa_select_topk writes them; row i sees blocks 0 .. i.
 *   DECODE:  idx [S, Hkv, dsa_decode_kmax] as dsa_decode writes it; every
 *            row sees the nB = ceil(seq_len / block) blocks; cnt NULL.
 *   PAGED:   idx [S, Hkv, dsa_decode_kmax] and cnt [S, Hkv] (or NULL) as
 *            dsa_paged_decode writes them, lengths [S] (device) the lengths
 *            it decoded; a row of sequence s sees ceil(lengths[s] / block)
 *            blocks (lengths clamped to 0 .. seq_len).
 * cnt NULL: a row's count is the length of its list before the first -1. */
#define DSA_LAYOUT_PREFILL 0
#define DSA_LAYOUT_DECODE 1
#define DSA_LAYOUT_PAGED 2

/* Errors: NULL idx/report (or cnt for PREFILL, lengths for PAGED), shape
 * errors (those of the call that wrote idx), an unknown layout. */
int dsa_check_block_selection(const dsa_shape* shape, int32_t layout, const int32_t* idx, const int32_t* cnt,
                              const int32_t* lengths, int64_t* report, void* stream);

/* The same for a token selection: idx [B, N, dsa_index_kmax] and cnt [B, N]
 * (or NULL) as dsa_index_topk or dsa_select_tokens write them; the row of
 * token t sees positions 0 .. t, the forced ones are 0 (DSA_FORCE_SINK) and
 * t (DSA_FORCE_DIAG), and its count is min(max(topk, F), t + 1). */
int dsa_check_token_selection(const dsa_index_shape* shape, const int32_t* idx, const int32_t* cnt, int64_t* report,
                              void* stream);

/* Static description of a status code. */
const char* dsa_status_str(int status);

/* Message for the last failing call on this thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
