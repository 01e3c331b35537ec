// Token-level lightning indexer and token-gather attention (gfx950).
//
// Method: "低成本高性能大模型实现路径：从架构创新到工程优化"
// (yunthe.com/news/806485.html), section 2.1 "轻量化索引器设计": an indexer of
// ReLU feature heads (16 index heads) decides, per query token, which 64
// key/value tokens matter; section 2.2 keeps the indexer's intermediates in
// low precision.  Here the score of earlier token s for query token t is
//   I[t, s] = sum_h w[t, h] * ReLU(qi[t, h] . ki[s])
// (bf16 MFMA, fp32 accumulation), each query token keeps its top-k tokens
// (sink and self forced, the best others by I, ties to the lower position),
// and every attention head attends over its token's kept key/value rows.
//
// Score tile (IndexRows, both score kernels): a workgroup holds 16 query
//   tokens, each wave 4 tokens = 2 tiles of 32 (token, index head) pairs.
//   Per 64-key tile (global -> LDS DMA, double-buffered, kswz rows): S =
//   Qi . K_tile^T on v_mfma_f32_32x32x16_bf16 (the wave's index query rows as
//   A in registers, key rows from LDS as B), so a lane's output holds one key
//   and 8 heads of each of two tokens; ReLU times the head weight is summed
//   over those in the lane and the other 8 heads' partial arrives by one
//   v_permlane32_swap per token pair.
// index_topk_kernel (fused scores + selection, no score array): units of 16
//   tokens x one chunk of key tiles; after each tile the scores are regrouped
//   so one register holds one token's 64 keys, and keys above the token's
//   running threshold join its LDS candidate list, which is compacted to a
//   new threshold when it fills (compact_candidates); at the end each list is
//   cut to its best m and written as the final row, or, for rows longer than
//   one chunk, as that chunk's list for index_merge_kernel.
// index_scores_kernel: the same tiles, every causal score stored (32
//   consecutive keys of a token per half-wave).  Token tiles run latest first
//   (they have the most key tiles).
// token_attn_kernel: one wave per (batch, token, KV head), KV-head-major over
//   XCD-contiguous workgroups (one KV head's rows per XCD L2).  The kept
//   positions arrive 64 at a time (one coalesced load, spread by lane
//   shuffles); per 32-token chunk the K rows load straight into registers as
//   MFMA A operands and the V rows go by DMA into a per-wave LDS tile (16
//   consecutive lanes per row, XOR-swizzled); Q K^T and P V both on
//   v_mfma_f32_16x16x32_bf16 with the heads as columns, P (rounded to bf16,
//   as in the block-sparse forward) passed from the S accumulators in
//   registers and V^T read back from the tile with ds_read_b64_tr_b16;
//   online softmax in fp32.
// select_tokens_fast_kernel: one wave per query-token row of up to 8192
//   scores.  The row is read in 256-token chunks, lane l holding tokens
//   4 l .. 4 l + 3 of each (one 16-byte load per lane, 1 KiB per wave
//   instruction; four chunks in flight).  Pass 1 keeps 8 group maxima per
//   lane, group k + 4 (c mod 2) for position k of chunk c, so a run of high
//   scores lands in many groups; the m-th largest of them (found exactly, no
//   early exit) is a lower bound t0 of the m-th largest candidate (the groups
//   are disjoint).  Pass 2 re-reads the chunks whose groups reach t0 and
//   compacts the candidates >= t0 -- usually about m -- into LDS in index
//   order (a prefix sum of the per-lane counts within a chunk); the threshold
//   search then runs on two keys per lane.  Rows it cannot finish (more than
//   64 to keep, or more than 128 candidates at or above t0) get cnt = -1 and
//   are completed by the general one-wave select.
#include "attn_common.hpp"
#include "decode_common.hpp"
#include "topk_row.hpp"

namespace dsa {
namespace {

template <int DI>
__device__ __forceinline__ void load_key_tile(const uint16_t* g, int row0, int n_rows, uint32_t lds_base, int wave,
                                              int lane) {
  constexpr int CH = DI / 8, RPI = 1024 / (2 * DI), LOADS = 64 * DI * 2 / 1024;
  static_assert(LOADS % 4 == 0, "tile loads split over 4 waves");
#pragma unroll
  for (int n = 0; n < LOADS / 4; ++n) {
    const int inst = wave + 4 * n;
    const int r = inst * RPI + lane / CH;
    const int c = (lane % CH) ^ kswz<DI>(r);
    const int row = min(row0 + r, n_rows - 1);
    dma16(g, (uint32_t)(row * DI + c * 8) * 2u, __builtin_amdgcn_readfirstlane(lds_base + inst * 1024));
  }
}

template <int DI>
__device__ __forceinline__ u32x4 key_frag(const LDS_AS uint16_t* tile, int r, int ks, int half) {
  const int c = (2 * ks + half) ^ kswz<DI>(r);
  return *reinterpret_cast<const LDS_AS u32x4*>(tile + r * DI + c * 8);
}

}  // namespace

// ReLU on the bit pattern: negative floats (and -0) have the sign bit set,
// so an integer max with 0 gives +0 for them and leaves the rest unchanged
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// ============================================================== index scores
// The index query rows, head weights and token numbers of a wave's four query
// tokens t0 + 4 wave .. t0 + 4 wave + 3, and the scores of a 64-key LDS tile
// against them.  A operands: row (lane % 32) of pair tile ct is the (token,
// index head) pair (t0 + 4 wave + 2 ct + (lane % 32) / 16, lane % 16).
template <int DI>
struct IndexRows {
  static constexpr int HI = 16, NKS = DI / 16;
  u32x4 qf[2][NKS];
  float wr[2][16];
  int tok[2];  // the token whose scores the lane ends with, per pair tile

  __device__ __forceinline__ void load(const uint16_t* qi, const float* wi, int64_t b, int N, int t0, int wave,
                                       int lane) {
    const int half = lane >> 5, i16 = lane & 15;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int tk = t0 + 4 * wave + 2 * ct + ((lane & 31) >> 4);
      const uint16_t* qrow = qi + ((b * N + min(tk, N - 1)) * HI + i16) * DI;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ct][ks] = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + 8 * half);
    }
    // Output register r of lane l holds key l % 32 and pair row
    // 8 (r / 4) + 4 half + r % 4: registers 0..7 are token 2 ct (heads
    // 4 half + r % 4 and 8 + 4 half + r % 4), 8..15 token 2 ct + 1, same
    // heads.  wr: the head weight of each register; the lane ends with the
    // score of token 2 ct + half.
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tr = t0 + 4 * wave + 2 * ct + (r >> 3);
        const int hd = 8 * ((r >> 2) & 1) + 4 * half + (r & 3);
        wr[ct][r] = wi[(b * N + min(tr, N - 1)) * HI + hd];
      }
      tok[ct] = t0 + 4 * wave + 2 * ct + half;
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(qf[ct][ks]));
  }

  // s[rt][ct]: the score of key 32 rt + lane % 32 of the tile for token tok[ct]
  __device__ __forceinline__ void tile(const LDS_AS uint16_t* tl, int lane, float (&s)[2][2]) const {
    const int half = lane >> 5;
    f32x16 acc[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const u32x4 a = key_frag<DI>(tl, rt * 32 + (lane & 31), ks, half);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qf[ct][ks]), as_bf16x8(a), acc[rt][ct], 0,
                                                                0, 0);
      }
    }
    // ReLU, head weight, sum over the heads: 8 of each token in the lane
    // (p0: token 2 ct, p1: token 2 ct + 1), the other 8 in lane l ^ 32.  One
    // swap of p0's upper 32 lanes with p1's lower 32 lanes leaves, in every
    // lane, the two partials of the token the lane keeps (2 ct + half).
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          p0 = __builtin_fmaf(relu_bits(acc[rt][ct][r]), wr[ct][r], p0);
          p1 = __builtin_fmaf(relu_bits(acc[rt][ct][8 + r]), wr[ct][8 + r], p1);
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
        s[rt][ct] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
    }
  }
};

template <int DI>
__global__ __launch_bounds__(256) void index_scores_kernel(const uint16_t* __restrict__ qi,
                                                           const uint16_t* __restrict__ ki,
                                                           const float* __restrict__ wi, float* __restrict__ scores,
                                                           int N, int tiles_per_b) {
  constexpr int KT = 64, TPB = 16;
  __shared__ __align__(1024) uint16_t kt_lds[2][KT * DI];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = blockIdx.x / tiles_per_b;
  const int tile = tiles_per_b - 1 - (int)(blockIdx.x % tiles_per_b);
  const int t0 = tile * TPB;
  const int n_kt = (min(t0 + TPB, N) - 1) / KT + 1;

  IndexRows<DI> rows;
  rows.load(qi, wi, b, N, t0, wave, lane);
  const uint16_t* kb = ki + b * (int64_t)N * DI;
  const uint32_t base[2] = {(uint32_t)(uintptr_t)(LDS_AS uint16_t*)kt_lds[0],
                            (uint32_t)(uintptr_t)(LDS_AS uint16_t*)kt_lds[1]};
  load_key_tile<DI>(kb, 0, N, base[0], wave, lane);

  for (int kt = 0; kt < n_kt; ++kt) {
    wait_vm<0>();
    __syncthreads();  // tile kt resident; every wave is done with tile kt - 1
    if (kt + 1 < n_kt) load_key_tile<DI>(kb, (kt + 1) * KT, N, base[(kt + 1) & 1], wave, lane);
    float s[2][2];
    rows.tile((const LDS_AS uint16_t*)kt_lds[kt & 1], lane, s);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const int key = kt * KT + rt * 32 + (lane & 31), t = rows.tok[ct];
        if (t < N && key <= t) scores[(b * N + t) * (int64_t)N + key] = s[rt][ct];
      }
  }
}

// ============================================================== fused scores + token selection
// Kept tokens of a row (ties to the lower position):
//   nv = t + 1 visible, the first na = min(anchors, nv) (the sink) and the
//   last nv - ws (ws = max(nv - window, na); the token itself) forced, and the
//   best m = min(max(topk, nf), nv) - nf of the candidates na <= s < ws.
struct TokenRow {
  int nv, na, ws, m;
  __device__ __forceinline__ TokenRow(int t, const TopkParams& p) {
    nv = t + 1;
    na = min(p.anchors, nv);
    ws = max(nv - p.window, na);
    const int nf = na + nv - ws;
    m = min(max(p.topk, nf), nv) - nf;
  }
};

// order_key's inverse: the float whose key is k (k > 0)
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Streaming top-m of one wave-held candidate list (CAP scores as fp32 bits
// and their positions in LDS, index order; 4 per lane, lane l holding entries
// 4 l .. 4 l + 3), ranked by their order keys.
// Keeps every entry >= T for the T the search ends at: the search starts at
// the common leading bits of the largest and smallest key and sets one more
// bit at a time while at least m entries stay at or above it, stopping as
// soon as at most `limit` remain.  If it runs out of bits first (T is then
// the m-th largest key exactly), the entries equal to T are cut to the
// lowest positions so that exactly m are kept.  Either way every dropped
// entry has m better ones (larger, or equal at a lower position), and so has
// every later (higher) position whose key does not exceed T: *thr becomes the
// acceptance threshold of later keys.  Returns the new count.
template <int CAP>
__device__ int compact_candidates(LDS_AS uint32_t* vals, LDS_AS int32_t* ids, int cnum, int m, int limit,
                                  uint32_t* thr, int lane) {
  static_assert(CAP == 256, "four entries per lane");
  const u32x4 fv = *reinterpret_cast<const LDS_AS u32x4*>(vals + 4 * lane);
  const u32x4 iv = *reinterpret_cast<const LDS_AS u32x4*>(ids + 4 * lane);
  uint32_t k[4];
  uint32_t mx = 0u, mn = ~0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    k[e] = 4 * lane + e < cnum ? order_key(__uint_as_float(fv[e])) : 0u;
    if (k[e]) {
      mx = max(mx, k[e]);
      mn = min(mn, k[e]);
    }
  }
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  const uint32_t x = mx ^ mn;
  int bit = x ? 31 - __builtin_clz(x) : -1;
  uint32_t T = x ? (mx & ~(uint32_t)(((uint64_t)2 << bit) - 1u)) : mx;
  int nT = cnum;
  for (; bit >= 0 && nT > limit; --bit) {
    const uint32_t trial = T | (1u << bit);
    const int c = wave_count_ge<4>(k, trial);
    if (c >= m) {
      T = trial;
      nT = c;
    }
  }
  const bool cut = nT > limit;
  const int n_gt = cut ? (T == ~0u ? 0 : wave_count_ge<4>(k, T + 1u)) : 0;
  int my_eq = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) my_eq += k[e] == T;
  int r = wave_incl_scan(my_eq) - my_eq;  // entries equal to T before this lane's
  bool keep[4];
  int mine = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    keep[e] = k[e] > T || (k[e] == T && (!cut || r < m - n_gt));
    r += k[e] == T;
    mine += keep[e];
  }
  const int incl = wave_incl_scan(mine);
  int pos = incl - mine;
  wave_lds_sync();  // every lane holds its entries before any is overwritten
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (keep[e]) {
      vals[pos] = fv[e];
      ids[pos] = (int32_t)iv[e];
      ++pos;
    }
  wave_lds_sync();
  *thr = max(*thr, T);
  return __builtin_amdgcn_readlane(incl, 63);
}

// One unit = 16 query tokens x one chunk of kct key tiles.  Chunk c of token
// tile tt exists for tt >= 4 c kct (the tile's keys reach past c kct tiles);
// units run chunk-major, latest tiles first.  Per 64-key tile the scores come
// from IndexRows::tile, regrouped so that one register holds one token's 64
// scores (key = lane); a key joins its token's candidate list (LDS, index
// order, the score's bits) when it is a candidate and its score exceeds the
// token's threshold (-inf until the first compaction; compared as floats,
// which orders like the keys).  Token state (counts, thresholds) is
// wave-uniform.  A list that
// may overflow on the next tile is compacted (compact_candidates, at most
// m + 32 left).  At the end each list is cut to its best m: a tile whose keys
// fit one chunk writes its final rows; otherwise each chunk's list goes to
// the workspace (as order keys) for index_merge_kernel.
template <int DI>
__global__ __launch_bounds__(256) void index_topk_kernel(const IndexTopkArgs a) {
  constexpr int KT = 64, TPB = 16, CAP = 256;
  __shared__ __align__(1024) uint16_t kt_lds[2][KT * DI];
  __shared__ __align__(16) uint32_t ckey[4][4][CAP];
  __shared__ __align__(16) int32_t cid[4][4][CAP];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t b = blockIdx.y;
  const int N = a.N;
  int u = blockIdx.x, c = 0;
  for (; c < a.nch; ++c) {
    const int uc = a.n_tt - 4 * c * a.kct;
    if (u < uc) break;
    u -= uc;
  }
  if (c >= a.nch) return;  // whole workgroup, before any barrier
  const int tt = a.n_tt - 1 - u;
  const int t0 = tt * TPB;
  const int n_kt = (min(t0 + TPB, N) - 1) / KT + 1;
  const int n_c = (n_kt - 1) / a.kct + 1;
  const int kt0 = c * a.kct, kt1 = min(kt0 + a.kct, n_kt);

  IndexRows<DI> rows;
  rows.load(a.qi, a.wi, b, N, t0, wave, lane);
  // per token j of the wave (t0 + 4 wave + j), all wave-uniform: candidate
  // range [lo, lo + span) (span 0: none), budget m, list length n, threshold
  // as an order key and as a float
  int lo[4], span[4], mr[4], n[4];
  uint32_t thr[4];
  float thf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + 4 * wave + j;
    const TokenRow tr(t, a.p);
    lo[j] = tr.na;
    span[j] = t < N && tr.m > 0 ? tr.ws - tr.na : 0;
    mr[j] = tr.m;
    n[j] = 0;
    thr[j] = 0u;
    thf[j] = -__builtin_inff();
  }
  const uint16_t* kb = a.ki + b * (int64_t)N * DI;
  const uint32_t base[2] = {(uint32_t)(uintptr_t)(LDS_AS uint16_t*)kt_lds[0],
                            (uint32_t)(uintptr_t)(LDS_AS uint16_t*)kt_lds[1]};
  load_key_tile<DI>(kb, kt0 * KT, N, base[0], wave, lane);

  for (int kt = kt0; kt < kt1; ++kt) {
    const int i = kt - kt0;
    wait_vm<0>();
    __syncthreads();  // tile i resident; every wave is done with tile i - 1
    if (kt + 1 < kt1) load_key_tile<DI>(kb, (kt + 1) * KT, N, base[(i + 1) & 1], wave, lane);
    float s[2][2];
    rows.tile((const LDS_AS uint16_t*)kt_lds[i & 1], lane, s);
    // s[rt][ct] holds keys 32 rt + lane % 32 of token 2 ct + half; swapping
    // s[0][ct]'s upper 32 lanes with s[1][ct]'s lower ones leaves token 2 ct's
    // 64 keys in one register and token 2 ct + 1's in the other, key = lane
    float v[4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s[0][ct]), __float_as_uint(s[1][ct]), false,
                                                       false);
      v[2 * ct] = __uint_as_float(sw[0]);
      v[2 * ct + 1] = __uint_as_float(sw[1]);
    }
    const int key = kt * KT + lane;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool take = (v[j] > thf[j]) & ((uint32_t)(key - lo[j]) < (uint32_t)span[j]);
      const uint64_t bal = __builtin_amdgcn_ballot_w64(take);
      if (take) {
        const int pos = n[j] + lanes_below(bal);
        ckey[wave][j][pos] = __float_as_uint(v[j]);
        cid[wave][j][pos] = key;
      }
      n[j] += __builtin_popcountll(bal);
    }
    // a list past CAP - 64 could overflow on the next tile
    if (max(max(n[0], n[1]), max(n[2], n[3])) > CAP - 64) {
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (n[j] > CAP - 64) {
          n[j] = compact_candidates<CAP>((LDS_AS uint32_t*)ckey[wave][j], (LDS_AS int32_t*)cid[wave][j], n[j], mr[j],
                                         mr[j] + 32, &thr[j], lane);
          thf[j] = key_float(thr[j]);
        }
    }
  }
  wave_lds_sync();

  // the best m of each list; then the final row or the chunk's list
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + 4 * wave + j;
    if (t >= N) break;
    int cs = n[j];
    const TokenRow tr(t, a.p);
    if (cs > tr.m) {
      uint32_t th = 0u;
      cs = compact_candidates<CAP>((LDS_AS uint32_t*)ckey[wave][j], (LDS_AS int32_t*)cid[wave][j], cs, tr.m, tr.m,
                                    &th, lane);
    }
    const int64_t row = b * N + t;
    if (n_c == 1) {
      int32_t* out = a.idx + row * a.kmax;
      for (int e = lane; e < tr.na; e += 64) out[e] = e;
      for (int e = lane; e < cs; e += 64) out[tr.na + e] = cid[wave][j][e];
      for (int e = lane; e < tr.nv - tr.ws; e += 64) out[tr.na + cs + e] = tr.ws + e;
      const int total = tr.na + cs + (tr.nv - tr.ws);
      for (int e = total + lane; e < a.kmax; e += 64) out[e] = -1;
      if (lane == 0) a.cnt[row] = total;
    } else {
      const int64_t slab = row * a.nch + c;
      for (int e = lane; e < cs; e += 64) {
        a.part_key[slab * a.mw + e] = order_key(__uint_as_float(ckey[wave][j][e]));
        a.part_idx[slab * a.mw + e] = cid[wave][j][e];
      }
      if (lane == 0) a.part_cnt[slab] = cs;
    }
  }
}

// One wave per row of a multi-chunk token tile (t >= t_first): the chunks'
// lists (each the best m of its keys, index order) concatenated in chunk
// order are in index order; lane l holds positions R l .. R l + R - 1 of the
// padded [n_c, mw] array.  The best m of the union are those of the row.
template <int R>
__global__ __launch_bounds__(256) void index_merge_kernel(const IndexTopkArgs a, int t_first, int B) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int N = a.N;
  const int64_t rows_per_b = N - t_first;
  const int64_t w = (int64_t)blockIdx.x * 4 + wave;
  if (w >= B * rows_per_b) return;  // whole wave; no workgroup barrier below
  const int64_t b = w / rows_per_b;
  const int t = t_first + (int)(w % rows_per_b);
  const int n_kt = (min((t / 16 + 1) * 16, N) - 1) / 64 + 1;
  const int n_c = (n_kt - 1) / a.kct + 1;
  const TokenRow tr(t, a.p);
  const int64_t row = b * N + t;
  const int64_t slab0 = row * a.nch;
  uint32_t k[R];
  int32_t id[R];
#pragma unroll
  for (int e = 0; e < R; ++e) {
    const int p = R * lane + e;
    const int sl = p / a.mw, j = p - sl * a.mw;
    const bool ok = sl < n_c && j < a.part_cnt[slab0 + min(sl, n_c - 1)];
    k[e] = ok ? a.part_key[(slab0 + sl) * a.mw + j] : 0u;
    id[e] = ok ? a.part_idx[(slab0 + sl) * a.mw + j] : 0;
  }
  const int total = wave_count_ge<R>(k, 1u);
  uint32_t T = 1u;
  bool cut = false;
  int n_gt = 0;
  if (total > tr.m) {
    uint32_t mx = 0u, mn = ~0u;
#pragma unroll
    for (int e = 0; e < R; ++e)
      if (k[e]) {
        mx = max(mx, k[e]);
        mn = min(mn, k[e]);
      }
    mx = wave_max_u32(mx);
    mn = wave_min_u32(mn);
    const uint32_t x = mx ^ mn;
    int bit = x ? 31 - __builtin_clz(x) : -1;
    T = x ? (mx & ~(uint32_t)(((uint64_t)2 << bit) - 1u)) : mx;
    int nT = total;
    for (; bit >= 0 && nT > tr.m; --bit) {
      const uint32_t trial = T | (1u << bit);
      const int cc = wave_count_ge<R>(k, trial);
      if (cc >= tr.m) {
        T = trial;
        nT = cc;
      }
    }
    cut = nT > tr.m;
    n_gt = cut ? (T == ~0u ? 0 : wave_count_ge<R>(k, T + 1u)) : 0;
  }
  int my_eq = 0;
#pragma unroll
  for (int e = 0; e < R; ++e) my_eq += k[e] == T;
  int r = wave_incl_scan(my_eq) - my_eq;
  bool keep[R];
  int mine = 0;
#pragma unroll
  for (int e = 0; e < R; ++e) {
    keep[e] = k[e] > T || (k[e] == T && (!cut || r < tr.m - n_gt));
    r += k[e] == T;
    mine += keep[e];
  }
  const int incl = wave_incl_scan(mine);
  const int nsel = __builtin_amdgcn_readlane(incl, 63);
  int32_t* out = a.idx + row * a.kmax;
  int pos = tr.na + incl - mine;
#pragma unroll
  for (int e = 0; e < R; ++e)
    if (keep[e]) out[pos++] = id[e];
  for (int e = lane; e < tr.na; e += 64) out[e] = e;
  for (int e = lane; e < tr.nv - tr.ws; e += 64) out[tr.na + nsel + e] = tr.ws + e;
  const int tot = tr.na + nsel + (tr.nv - tr.ws);
  for (int e = tot + lane; e < a.kmax; e += 64) out[e] = -1;
  if (lane == 0) a.cnt[row] = tot;
}

// ============================================================== token attention
// One wave per (batch, token, KV head): the G query heads of the token attend
// over its kept tokens in 32-key chunks (v_mfma_f32_16x16x32_bf16 for both
// products, heads as the 16 N columns, zero past G).
//   S = K Q^T: K rows are A operands loaded straight into registers (lane l:
//     key l % 16 of a 16-key half, 16 bytes at dims ks * 32 + 8 (l / 16));
//     the output puts head l % 16 in the lane and keys 16 sb + 4 (l / 16) + j
//     in its slots, so row max and sum are in-lane plus two xor shuffles.
//   O^T += V^T P^T: P leaves the S accumulators already in B-operand order
//     (slot 4 sb + j <-> key 16 sb + 4 (l / 16) + j); the V rows go by DMA
//     into this wave's LDS tile and come back as the V^T A operand through
//     ds_read_b64_tr_b16 (within 16 lanes, lane i slot j receives element i % 4
//     of the 8-byte piece of source lane 4 j + i / 4), the source lanes of
//     16-lane group g reading keys 4 g + 16 sg + j, which is the same key order.
// The V tile's 16-byte chunks are XOR-swizzled by row (vtsw) so that the 32
// lanes of two groups read eight distinct 32-byte bank ranges.
template <int D>
__device__ __forceinline__ int vtsw(int r) {
  return D == 128 ? 2 * ((r & 3) + 4 * ((r >> 2) & 1)) : 2 * (((r >> 1) & 1) + 2 * ((r >> 2) & 1));
}

template <int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
void token_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                       const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
                       const int32_t* __restrict__ cnt, uint16_t* __restrict__ o, float* __restrict__ lse,
                       int Hkv, int N, int kmax, float scale_log2, int64_t n_waves) {
  static_assert(G <= 16, "heads are the 16 MFMA columns");
  constexpr int CK = 32;                                   // keys per chunk
  constexpr int CH = D / 8, RPI = 64 / CH, NL = CK / RPI;  // V DMA: lanes per row, rows per DMA, DMAs per chunk
  constexpr int NKS = D / 32, NDB = D / 16;                // k-steps of Q K^T, 16-dim blocks of O
  __shared__ __align__(1024) uint16_t vtile[4][CK * D];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, lq = lane >> 4;
  // KV-head-major over XCD-contiguous workgroup ranges: the waves of one XCD
  // gather from one KV head's rows, which then stay in that XCD's L2
  const int64_t w = (int64_t)xcd_logical_id(blockIdx.x, gridDim.x) * 4 + wave;
  if (w >= n_waves) return;  // whole wave; no workgroup barrier below
  const int64_t BN = n_waves / Hkv;
  const int g = (int)(w / BN);
  const int64_t bt = w % BN;  // b * N + t
  const int t = (int)(bt % N);
  const int64_t b = bt / N;
  const int Hq = Hkv * G;
  const int nk = min(max(cnt[bt], 0), kmax);
  const int32_t* row = idx + bt * kmax;
  const uint16_t* kb = k + (b * Hkv + g) * (int64_t)N * D;
  const uint16_t* vb = v + (b * Hkv + g) * (int64_t)N * D;
  const uint16_t* q0 = q + ((b * Hq + g * G) * (int64_t)N + t) * D;  // head hh's row at q0 + hh N D
  const LDS_AS uint16_t* vt = (const LDS_AS uint16_t*)(vtile[wave]);
  const uint32_t vt_base = (uint32_t)(uintptr_t)vt;

  // B operand of S = K Q^T: column n is head n (zero past G), slots <-> dims
  // ks * 32 + 8 lq + e
  u32x4 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = (u32x4){0, 0, 0, 0};
    if (n < G) qf[ks] = *reinterpret_cast<const u32x4*>(q0 + (int64_t)n * N * D + ks * 32 + 8 * lq);
  }
  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = (f32x4){0, 0, 0, 0};
  const float NEG_INF = -__builtin_inff();
  float m_run = NEG_INF, l_run = 0.f;  // head n's state, in log2 units

  // kept positions base .. base + 63, one per lane; positions past nk repeat
  // the last kept token (a finite row whose weight is masked to 0)
  auto ids = [&](int base) {
    const int p = min(base + lane, nk - 1);
    return min(max(row[p], 0), N - 1);
  };
  const int nch = (nk + CK - 1) / CK;
  int iv = 0;
  for (int c = 0; c < nch; ++c) {
    const int cc = c & 1;  // chunk within the 64 positions in iv
    if (cc == 0) iv = ids(c * CK);
    // V rows -> LDS: each DMA brings RPI whole rows (CH consecutive lanes per
    // row, every request covering full cache lines), lane l landing in slot l
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int rr = i * RPI + lane / CH;
      const int key = __shfl(iv, 32 * cc + rr, 64);
      const int ch = (lane % CH) ^ vtsw<D>(rr);
      dma16(vb, (uint32_t)(key * D + ch * 8) * 2u, __builtin_amdgcn_readfirstlane(vt_base + i * 1024));
    }
    // K rows as A operands
    u32x4 kf[2][NKS];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int key = __shfl(iv, 32 * cc + 16 * sb + n, 64);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        kf[sb][ks] = *reinterpret_cast<const u32x4*>(kb + (int64_t)key * D + ks * 32 + 8 * lq);
    }
    f32x4 sc[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      sc[sb] = (f32x4){0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        sc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[sb][ks]), as_bf16x8(qf[ks]), sc[sb], 0, 0, 0);
    }
    // logits in log2 units, positions past nk masked; running max and sum
    float mloc = NEG_INF;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int pos = c * CK + 16 * sb + 4 * lq + j;
        const float x = pos < nk ? sc[sb][j] * scale_log2 : NEG_INF;
        sc[sb][j] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);  // finite: a chunk holds a position below nk
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
    u32x4 pf;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      float p4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p4[j] = __builtin_amdgcn_exp2f(sc[sb][j] - m_run);
        lsum += p4[j];
      }
      const bf16x2_t lo = {(__bf16)p4[0], (__bf16)p4[1]};
      const bf16x2_t hi = {(__bf16)p4[2], (__bf16)p4[3]};
      pf[2 * sb] = __builtin_bit_cast(uint32_t, lo);
      pf[2 * sb + 1] = __builtin_bit_cast(uint32_t, hi);
    }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    // ---- O^T += V^T P^T, the V^T operand by transposed reads of the tile
    wait_vm<0>();  // this wave's V DMAs have landed
    const int src = lane & 15;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      u32x4 va;
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        const int r = 4 * lq + 16 * sg + (src >> 2);  // key row of the chunk
        const int d0 = db * 16 + 4 * (src & 3);       // first of this source lane's 4 dims
        const int ch = (d0 >> 3) ^ vtsw<D>(r);
        const LDS_AS char* addr = reinterpret_cast<const LDS_AS char*>(vt + r * D + ch * 8) + (d0 & 7) * 2;
        const i16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)addr);
        const u32x2 w2 = __builtin_bit_cast(u32x2, v4);
        va[2 * sg] = w2[0];
        va[2 * sg + 1] = w2[1];
      }
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pf), acc[db], 0, 0, 0);
    }
  }

  // O = acc / l (bf16): lane (n, lq) holds head n's dims db * 16 + 4 lq + j;
  // LSE = (m + log2 l) ln 2
  if (n < G) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    uint16_t* orow = o + ((b * Hq + g * G + n) * (int64_t)N + t) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const bf16x2_t lo = {(__bf16)(acc[db][0] * inv), (__bf16)(acc[db][1] * inv)};
      const bf16x2_t hi = {(__bf16)(acc[db][2] * inv), (__bf16)(acc[db][3] * inv)};
      u32x2 w2;
      w2[0] = __builtin_bit_cast(uint32_t, lo);
      w2[1] = __builtin_bit_cast(uint32_t, hi);
      *reinterpret_cast<u32x2*>(orow + db * 16 + 4 * lq) = w2;
    }
    if (lse && lq == 0)
      lse[(b * Hq + g * G + n) * (int64_t)N + t] =
          l_run > 0.f ? (m_run + __log2f(l_run)) * 0.6931471805599453f : -__builtin_inff();
  }
}

// ============================================================== token selection
__global__ __launch_bounds__(256) void select_tokens_fast_kernel(const float* __restrict__ scores,
                                                                 int32_t* __restrict__ idx, int32_t* __restrict__ cnt,
                                                                 int64_t n_rows, int N, TopkParams p, int kmax) {
  __shared__ uint32_t lds_key[4][128];
  __shared__ int32_t lds_idx[4][128];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= n_rows) return;  // whole wave; no workgroup barrier below
  const int nv = (int)(row % N) + 1;
  const float* srow = scores + row * (int64_t)N;
  int32_t* out = idx + row * (int64_t)kmax;
  const int na = min(p.anchors, nv);
  const int ws = max(nv - p.window, na);
  const int nf = na + (nv - ws);
  const int budget = min(max(p.topk, nf), nv);
  const int m = budget - nf;
  const int ncand = nv - nf;
  if (m >= ncand || m <= 0) {  // every visible token, or the forced ones only
    const int total = m <= 0 ? nf : nv;
    for (int e = lane; e < total; e += 64) out[e] = m <= 0 ? (e < na ? e : ws + (e - na)) : e;
    for (int e = total + lane; e < kmax; e += 64) out[e] = -1;
    if (lane == 0) cnt[row] = total;
    return;
  }
  if (m > 64) {
    if (lane == 0) cnt[row] = -1;
    return;
  }
  // token j = 256 c + 4 lane + k; a 16-byte load when the four are
  // candidates and the row is 16-byte aligned, else one load per candidate
  constexpr int CB = 4;  // chunks per batch
  const int c_lo = (na / 256) & ~(CB - 1), c_hi = (ws - 1) / 256;
  const bool aligned = (N & 3) == 0;
  auto load4 = [&](int c, uint32_t (&kv)[4], bool want) {
    const int j0 = 256 * c + 4 * lane;
    if (want && aligned && j0 >= na && j0 + 3 < ws) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(srow + j0);
#pragma unroll
      for (int k = 0; k < 4; ++k) kv[k] = order_key(v[k]);
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) kv[k] = (want && j0 + k >= na && j0 + k < ws) ? order_key(srow[j0 + k]) : 0u;
    }
  };
  // pass 1: group maxima of the candidate keys (0 = no candidate)
  uint32_t gmax[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) gmax[g] = 0u;
  for (int c0 = c_lo; c0 <= c_hi; c0 += CB) {
    uint32_t kv[CB][4];
#pragma unroll
    for (int u = 0; u < CB; ++u) load4(c0 + u, kv[u], true);
#pragma unroll
    for (int u = 0; u < CB; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) gmax[k + 4 * (u & 1)] = max(gmax[k + 4 * (u & 1)], kv[u][k]);
  }
  bool ex;
  const uint32_t t0 = wave_kth_largest<8, false>(gmax, m, &ex);  // the m-th largest group maximum
  // pass 2: compact the candidates >= t0 in index order; a lane reads a chunk
  // again only when one of its groups there reaches t0
  int ns = 0;
  if (t0 > 0u) {
    for (int c0 = c_lo; c0 <= c_hi; c0 += CB) {
      uint32_t kv[CB][4];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const int gb = 4 * (u & 1);
        load4(c0 + u, kv[u], max(max(gmax[gb], gmax[gb + 1]), max(gmax[gb + 2], gmax[gb + 3])) >= t0);
      }
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        int mine = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) mine += kv[u][k] >= t0;
        const int incl = wave_incl_scan(mine);
        int pos = ns + incl - mine;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (kv[u][k] >= t0) {
            if (pos < 128) {
              lds_key[wave][pos] = kv[u][k];
              lds_idx[wave][pos] = 256 * (c0 + u) + 4 * lane + k;
            }
            ++pos;
          }
        ns += __builtin_amdgcn_readlane(incl, 63);
      }
    }
  }
  if (t0 == 0u || ns > 128) {
    if (lane == 0) cnt[row] = -1;
    return;
  }
  wave_lds_sync();
  const bool ok0 = lane < ns, ok1 = lane + 64 < ns;
  const uint32_t k0 = ok0 ? lds_key[wave][lane] : 0u, k1 = ok1 ? lds_key[wave][64 + lane] : 0u;
  const int i0 = ok0 ? lds_idx[wave][lane] : -1, i1 = ok1 ? lds_idx[wave][64 + lane] : -1;
  bool exact;
  const uint32_t kk[2] = {k0, k1};
  const uint32_t T = wave_kth_largest<2>(kk, m, &exact);
  const int n_gt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok0 && k0 > T)) +
                   __builtin_popcountll(__builtin_amdgcn_ballot_w64(ok1 && k1 > T));
  const uint64_t eq0 = __builtin_amdgcn_ballot_w64(ok0 && k0 == T);
  const uint64_t eq1 = __builtin_amdgcn_ballot_w64(ok1 && k1 == T);
  const int take_eq = exact ? 128 : m - n_gt;
  const bool s0 = ok0 && (k0 > T || (k0 == T && lanes_below(eq0) < take_eq));
  const bool s1 = ok1 && (k1 > T || (k1 == T && __builtin_popcountll(eq0) + lanes_below(eq1) < take_eq));
  const uint64_t sm0 = __builtin_amdgcn_ballot_w64(s0), sm1 = __builtin_amdgcn_ballot_w64(s1);
  const int nsel = __builtin_popcountll(sm0) + __builtin_popcountll(sm1);
  if (s0) out[na + lanes_below(sm0)] = i0;
  if (s1) out[na + __builtin_popcountll(sm0) + lanes_below(sm1)] = i1;
  for (int e = lane; e < na; e += 64) out[e] = e;
  for (int e = lane; e < nv - ws; e += 64) out[na + nsel + e] = ws + e;
  const int total = na + nsel + (nv - ws);
  for (int e = total + lane; e < kmax; e += 64) out[e] = -1;
  if (lane == 0) cnt[row] = total;
}

// ============================================================== launch
hipError_t launch_index_scores(const uint16_t* qi, const uint16_t* ki, const float* wi, float* scores, int B, int N,
                               int di, hipStream_t stream) {
  if (B == 0 || N == 0) return hipSuccess;
  const int tiles = (N + 15) / 16;
  const dim3 grid((uint32_t)((int64_t)B * tiles)), blk(256);
  if (di == 64) hipLaunchKernelGGL(index_scores_kernel<64>, grid, blk, 0, stream, qi, ki, wi, scores, N, tiles);
  else hipLaunchKernelGGL(index_scores_kernel<128>, grid, blk, 0, stream, qi, ki, wi, scores, N, tiles);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_token_attn_d(const TokenAttnArgs& a, hipStream_t stream) {
  const int64_t n_waves = (int64_t)a.B * a.N * a.Hkv;
  if (n_waves == 0) return hipSuccess;
  const dim3 grid((uint32_t)((n_waves + 3) / 4)), blk(256);
#define DSA_TOKEN_ATTN(GG)                                                                                          \
  hipLaunchKernelGGL((token_attn_kernel<D, GG>), grid, blk, 0, stream, a.q, a.k, a.v, a.idx, a.cnt, a.o, a.lse, a.Hkv, \
                     a.N, a.kmax, a.scale_log2, n_waves)
  switch (a.Hq / a.Hkv) {
    case 1: DSA_TOKEN_ATTN(1); break;
    case 2: DSA_TOKEN_ATTN(2); break;
    case 4: DSA_TOKEN_ATTN(4); break;
    case 8: DSA_TOKEN_ATTN(8); break;
    default: return hipErrorInvalidValue;
  }
#undef DSA_TOKEN_ATTN
  return hipGetLastError();
}

hipError_t launch_index_topk(const uint16_t* qi, const uint16_t* ki, const float* wi, int32_t* idx, int32_t* cnt,
                             void* ws, int B, int N, int di, TopkParams p, int kmax, hipStream_t stream) {
  if (B == 0 || N == 0) return hipSuccess;
  if (kmax > INDEX_TOPK_MAX_KEEP) return hipErrorInvalidValue;
  const IndexTopkPlan pl = plan_index_topk(B, N, kmax);
  IndexTopkArgs a{};
  a.qi = qi;
  a.ki = ki;
  a.wi = wi;
  a.idx = idx;
  a.cnt = cnt;
  const size_t n_slab = (size_t)B * N * pl.nch;
  a.part_key = pl.nch > 1 ? static_cast<uint32_t*>(ws) : nullptr;
  a.part_idx = pl.nch > 1 ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + n_slab * pl.mw * 4) : nullptr;
  a.part_cnt = pl.nch > 1 ? reinterpret_cast<int32_t*>(static_cast<char*>(ws) + n_slab * pl.mw * 8) : nullptr;
  a.N = N;
  a.n_tt = (N + 15) / 16;
  a.kct = pl.kct;
  a.nch = pl.nch;
  a.mw = pl.mw;
  a.kmax = kmax;
  a.p = p;
  int64_t units = 0;
  for (int c = 0; c < pl.nch; ++c) units += a.n_tt - 4 * c * pl.kct;
  const dim3 grid((uint32_t)units, (uint32_t)B), blk(256);
  if (di == 64) hipLaunchKernelGGL(index_topk_kernel<64>, grid, blk, 0, stream, a);
  else hipLaunchKernelGGL(index_topk_kernel<128>, grid, blk, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.nch == 1) return e;
  const int t_first = 64 * pl.kct;
  const int64_t rows = (int64_t)B * (N - t_first);
  const dim3 mgrid((uint32_t)((rows + 3) / 4));
  const int pos = pl.nch * pl.mw;
  if (pos <= 128) hipLaunchKernelGGL(index_merge_kernel<2>, mgrid, blk, 0, stream, a, t_first, B);
  else if (pos <= 256) hipLaunchKernelGGL(index_merge_kernel<4>, mgrid, blk, 0, stream, a, t_first, B);
  else if (pos <= 512) hipLaunchKernelGGL(index_merge_kernel<8>, mgrid, blk, 0, stream, a, t_first, B);
  else hipLaunchKernelGGL(index_merge_kernel<16>, mgrid, blk, 0, stream, a, t_first, B);
  return hipGetLastError();
}

hipError_t launch_select_tokens(const float* scores, int32_t* idx, int32_t* cnt, int64_t n_rows, int N, TopkParams p,
                                int kmax, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  if (N > 64 * 128) return hipErrorInvalidValue;
  const int nf = (p.anchors > 0 ? 1 : 0) + (p.window > 0 ? 1 : 0);
  if (p.topk - nf > 64)  // the fast path cannot take these rows: general select for all
    return launch_select_topk(scores, idx, cnt, n_rows, N, N, true, p, kmax, stream);
  hipLaunchKernelGGL(select_tokens_fast_kernel, dim3((uint32_t)((n_rows + 3) / 4)), dim3(256), 0, stream, scores, idx,
                     cnt, n_rows, N, p, kmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_select_marked(scores, idx, cnt, n_rows, N, p, kmax, stream);
}

hipError_t launch_token_attn(const TokenAttnArgs& a, int d, hipStream_t stream) {
  if (a.B == 0 || a.N == 0) return hipSuccess;
  return d == 64 ? launch_token_attn_d<64>(a, stream) : launch_token_attn_d<128>(a, stream);
}

}  // namespace dsa
