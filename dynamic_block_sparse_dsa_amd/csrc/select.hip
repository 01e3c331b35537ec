// Block selection kernels: block means, causal block scores, top-k select.
//
// Method sources (by page and section):
//   "dynamic sparse attention explainer" (zblog.xzdbk.com/559.html):
//     "基于Top-k选择的局部-全局混合" -- per query keep the k best-scoring keys,
//     plus global and local anchors; "硬件友好的稀疏计算实现" -- decide per
//     fixed-size block; "前沿方向" -- a GQA group shares its KV cache and so
//     one selection.
//   "稀疏注意力 vs Flash Attention v2" (pnsm.cn/news/1249548.html), section 1:
//     content-aware top-k ranks keys by query-key similarity.
//   DeepSeek NSA article (pnsm.cn/news/1939904.html), section 2.2: the
//     routing decision is made in fp32.
// The block statistic is mean(Q tile) . mean(K tile) / sqrt(d), so all three
// kernels work in fp32 on the block means.
#include "dsa_internal.hpp"
#include "topk_row.hpp"

namespace dsa {

// ============================================================== block means
// The mean of one block is computed by one 64-lane wave in a fixed order:
// lane l owns the 16-byte chunk c = l % CH of the row (CH = D/8 chunks) and
// the row group r = l / CH (RG = 64/CH groups); it sums the rows r, r + RG,
// r + 2 RG, ... of the block in fp32, then lane (0, c) adds the RG partial
// sums in group order and divides by the number of real rows.  Every kernel
// that pools a block (the means kernel and the fused score kernel) uses this
// function, so both give the same bits.
template <int D>
__device__ __forceinline__ void wave_block_mean(const uint16_t* __restrict__ rows0, int rows, int lane, float* out8) {
  constexpr int CH = D / 8, RG = 64 / CH;
  const int c = lane % CH, rg = lane / CH;
  const uint16_t* base = rows0 + c * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 8
  for (int r = rg; r < rows; r += RG) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(base + (int64_t)r * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_lo(w[e]);
      acc[2 * e + 1] += bf16_hi(w[e]);
    }
  }
  const float rows_f = (float)rows;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float s = __shfl(acc[e], c, 64);
#pragma unroll
    for (int g = 1; g < RG; ++g) s += __shfl(acc[e], c + g * CH, 64);
    out8[e] = s / rows_f;
  }
}

// One wave per (unit, block); four waves per workgroup.  Two tensors in one
// launch: the n0 * nB blocks of x0, then those of x1.
template <int D>
__global__ __launch_bounds__(256) void block_means_kernel(const uint16_t* __restrict__ x0, float* __restrict__ xbar0,
                                                          int64_t n0, const uint16_t* __restrict__ x1,
                                                          float* __restrict__ xbar1, int64_t n_total, int N,
                                                          int block, int nB) {
  constexpr int CH = D / 8;
  const int lane = threadIdx.x & 63;
  int64_t wb = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (unit, block) of this wave
  if (wb >= n_total) return;
  const uint16_t* x = x0;
  float* xbar = xbar0;
  if (wb >= n0 * nB) {
    wb -= n0 * nB;
    x = x1;
    xbar = xbar1;
  }
  const int64_t unit = wb / nB;
  const int j = (int)(wb % nB);
  const int r0 = j * block;
  float m[8];
  wave_block_mean<D>(x + (unit * N + r0) * (int64_t)D, min(block, N - r0), lane, m);
  if (lane < CH) {
    float* dst = xbar + (unit * nB + j) * (int64_t)D + lane * 8;
    *reinterpret_cast<f32x4*>(dst) = (f32x4){m[0], m[1], m[2], m[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = (f32x4){m[4], m[5], m[6], m[7]};
  }
}

hipError_t launch_block_means2(const uint16_t* x0, float* xbar0, int64_t n0, const uint16_t* x1, float* xbar1,
                               int64_t n1, int N, int d, int block, hipStream_t stream) {
  const int nB = (N + block - 1) / block;
  const int64_t n_total = (n0 + n1) * nB;
  if (n_total == 0) return hipSuccess;
  const uint32_t n_wg = (uint32_t)((n_total + 3) / 4);
  if (d == 64)
    hipLaunchKernelGGL(block_means_kernel<64>, dim3(n_wg), dim3(256), 0, stream, x0, xbar0, n0, x1, xbar1, n_total,
                       N, block, nB);
  else
    hipLaunchKernelGGL(block_means_kernel<128>, dim3(n_wg), dim3(256), 0, stream, x0, xbar0, n0, x1, xbar1, n_total,
                       N, block, nB);
  return hipGetLastError();
}

hipError_t launch_block_means(const uint16_t* x, float* xbar, int64_t n_units, int N, int d, int block,
                              hipStream_t stream) {
  return launch_block_means2(x, xbar, n_units, nullptr, nullptr, 0, N, d, block, stream);
}

// ============================================================== block scores
// One 256-thread workgroup per TS x TS tile of the score matrix of one (batch,
// KV head): thread (ty, tx) owns rows ty + 16 r and columns tx + 16 c
// (r, c < TS / 16).  Both tiles of means are staged whole in LDS (row pitch
// D+4 floats: the float4 reads of 16 K rows hit distinct bank groups, the Q
// reads are broadcasts); the K tile and the first Q tile are fetched together;
// every head of the group is scored against the K tile and the max is kept.
// Tiles strictly above the diagonal are -inf.  Each score is one fp32 FMA
// chain over the dims in order, so the tile size changes no bit; 64-row tiles
// (4 x 4 scores per thread) read half the LDS bytes per score of 32-row ones
// and serve the large score matrices, 32-row tiles the small ones (more
// workgroups).
template <int D, int TS>
__global__ __launch_bounds__(256) void block_scores_kernel(const float* __restrict__ qbar,
                                                           const float* __restrict__ kbar, float* __restrict__ scores,
                                                           int Hq, int Hkv, int nB, float scale, int n_tiles) {
  constexpr int PITCH = D + 4;  // rows 16-byte aligned, one bank group apart: conflict-free float4 reads
  constexpr int RT = TS / 16;   // rows (and columns) per thread
  constexpr int PER_T = TS * D / 4 / 256;  // float4 pieces of a tile per thread
  __shared__ __align__(16) float qs[TS][PITCH];
  __shared__ __align__(16) float ks[TS][PITCH];
  const int per_unit = n_tiles * n_tiles;
  const int64_t unit = blockIdx.x / per_unit;  // b * Hkv + g
  const int tile = blockIdx.x % per_unit;
  const int ti = tile / n_tiles, tj = tile % n_tiles;
  const int t = threadIdx.x, tx = t % 16, ty = t / 16;
  const int i0 = ti * TS, j0 = tj * TS;
  float* out = scores + unit * (int64_t)nB * nB;
  const float NEG_INF = -__builtin_inff();
  if (tj > ti) {
    for (int e = t; e < TS * TS; e += 256) {
      const int i = i0 + e / TS, j = j0 + e % TS;
      if (i < nB && j < nB) out[(int64_t)i * nB + j] = NEG_INF;
    }
    return;
  }
  const int G = Hq / Hkv;
  const int64_t b = unit / Hkv, g = unit % Hkv;
  const float* kb = kbar + unit * (int64_t)nB * D;
  // a TS-row tile of means: global -> registers (rows past nB read as 0), then LDS
  auto fetch = [&](const float* src, int r0, f32x4 (&v)[PER_T]) {
#pragma unroll
    for (int n = 0; n < PER_T; ++n) {
      const int e = t + 256 * n, r = e / (D / 4), c = e % (D / 4);
      v[n] = (f32x4){0, 0, 0, 0};
      if (r0 + r < nB) v[n] = *reinterpret_cast<const f32x4*>(src + (int64_t)(r0 + r) * D + 4 * c);
    }
  };
  auto stash = [&](float (*dst)[PITCH], const f32x4 (&v)[PER_T]) {
#pragma unroll
    for (int n = 0; n < PER_T; ++n) {
      const int e = t + 256 * n, r = e / (D / 4), c = e % (D / 4);
      *reinterpret_cast<f32x4*>(&dst[r][4 * c]) = v[n];
    }
  };
  float best[RT][RT];
  for (int hh = 0; hh < G; ++hh) {
    const float* qb = qbar + ((b * Hq) + g * G + hh) * (int64_t)nB * D;
    f32x4 qv[PER_T];
    if (hh == 0) {  // the K tile and the first head's Q tile are fetched together
      f32x4 kv[PER_T];
      fetch(kb, j0, kv);
      fetch(qb, i0, qv);
      stash(ks, kv);
    } else {
      fetch(qb, i0, qv);
      __syncthreads();  // previous head's reads of qs are done
    }
    stash(qs, qv);
    __syncthreads();
    float acc[RT][RT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < RT; ++c) acc[r][c] = 0.f;
#pragma unroll 4
    for (int dd = 0; dd < D; dd += 4) {
      f32x4 av[RT], bv[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) av[r] = *reinterpret_cast<const f32x4*>(&qs[ty + 16 * r][dd]);
#pragma unroll
      for (int c = 0; c < RT; ++c) bv[c] = *reinterpret_cast<const f32x4*>(&ks[tx + 16 * c][dd]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int r = 0; r < RT; ++r)
#pragma unroll
          for (int c = 0; c < RT; ++c) acc[r][c] = __builtin_fmaf(av[r][e], bv[c][e], acc[r][c]);
    }
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int c = 0; c < RT; ++c) {
        const float sc = acc[r][c] * scale;
        best[r][c] = (hh == 0) ? sc : fmaxf(best[r][c], sc);
      }
  }
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int c = 0; c < RT; ++c) {
      const int i = i0 + ty + 16 * r, j = j0 + tx + 16 * c;
      if (i < nB && j < nB) out[(int64_t)i * nB + j] = (j <= i) ? best[r][c] : NEG_INF;
    }
}

// 64-row tiles once the matrix has at least 8 of them per side
hipError_t launch_block_scores(const float* qbar, const float* kbar, float* scores, int B, int Hq, int Hkv, int nB,
                               int d, float scale, hipStream_t stream) {
  const bool big = nB >= 512;
  const int ts = big ? 64 : 32;
  const int n_tiles = (nB + ts - 1) / ts;
  const int64_t n_wg = (int64_t)B * Hkv * n_tiles * n_tiles;
  if (n_wg == 0) return hipSuccess;
#define DSA_SCORES(DD, TT)                                                                                        \
  hipLaunchKernelGGL((block_scores_kernel<DD, TT>), dim3((uint32_t)n_wg), dim3(256), 0, stream, qbar, kbar, scores, \
                     Hq, Hkv, nB, scale, n_tiles)
  if (d == 64) {
    if (big) DSA_SCORES(64, 64);
    else DSA_SCORES(64, 32);
  } else {
    if (big) DSA_SCORES(128, 64);
    else DSA_SCORES(128, 32);
  }
#undef DSA_SCORES
  return hipGetLastError();
}

// ============================================================== scores from Q, K
// Block scores straight from the bf16 Q and K, with no workspace.  One
// 256-thread workgroup per (batch, KV head, strip of T query blocks, strip of
// T key blocks), key strip <= query strip.  The workgroup pools its query
// strip for up to HC heads at a time into LDS (wave_block_mean: the bits of
// block_means_kernel), then for every 32-block tile of its key strip pools
// those key blocks into LDS and scores each (query block, key block) pair with
// the dot-product order of block_scores_kernel, keeping the max over the
// heads.  So the result equals block_scores_kernel on the block means, bit for
// bit.  A query strip of T blocks is re-pooled once per key strip and a key
// tile once per query strip (and head chunk): about nB / T reads of Q and K
// in all, against one read for the means + scores path, which dsa_prefill
// takes since it has a workspace.
template <int D, int HC>
__global__ __launch_bounds__(256) void pooled_scores_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k,
                                                            float* __restrict__ scores, int Hq, int Hkv, int N,
                                                            int block, int nB, int T, int n_strips, float scale) {
  constexpr int PITCH = D + 4;
  constexpr int CH = D / 8;
  __shared__ __align__(16) float qs[256][PITCH];  // row hh * T + i: head hh of the chunk, query block qb0 + i
  __shared__ __align__(16) float ks[32][PITCH];
  const int n_pairs = n_strips * (n_strips + 1) / 2;
  const int64_t unit = blockIdx.x / n_pairs;  // b * Hkv + g
  const int pair = (int)(blockIdx.x % n_pairs);
  int si = 0;
  while ((si + 1) * (si + 2) / 2 <= pair) ++si;
  const int sj = pair - si * (si + 1) / 2;
  const int G = Hq / Hkv;
  const int64_t b = unit / Hkv, g = unit % Hkv;
  const int qb0 = si * T, kb0 = sj * T;
  const int nq = min(T, nB - qb0);                  // query blocks of the strip
  const int k_end = min(kb0 + T, qb0 + nq);        // key blocks kb0 .. k_end - 1 can be visible
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, tx = t % 16, ty = t / 16;
  float* out = scores + unit * (int64_t)nB * nB;
  const float NEG_INF = -__builtin_inff();
  const uint16_t* kunit = k + unit * (int64_t)N * D;

  // -inf where no tile below computes: key columns past the key strip's
  // visible end (diagonal strip only) and 32x32 tiles wholly above the
  // diagonal; disjoint from what the tiles write
  if (si == sj) {
    const int ncols = nB - qb0;
    for (int64_t e = t; e < (int64_t)nq * ncols; e += 256) {
      const int ii = (int)(e / ncols), j = qb0 + (int)(e % ncols);
      const int qt = ii & ~31, i_hi = qb0 + min(qt + 32, nq) - 1;
      const int kt = qb0 + ((j - qb0) & ~31);
      if (j >= k_end || kt > i_hi) out[(int64_t)(qb0 + ii) * nB + j] = NEG_INF;
    }
  }

  for (int hc = 0; hc < G; hc += HC) {
    const int nh = min(HC, G - hc);
    __syncthreads();  // the previous chunk is done reading qs
    for (int e = wave; e < nh * nq; e += 4) {
      const int hh = e / nq, i = e % nq;
      const int64_t h = g * G + hc + hh;
      const int r0 = (qb0 + i) * block;
      float m[8];
      wave_block_mean<D>(q + ((b * Hq + h) * N + r0) * (int64_t)D, min(block, N - r0), lane, m);
      if (lane < CH) {
        *reinterpret_cast<f32x4*>(&qs[hh * T + i][lane * 8]) = (f32x4){m[0], m[1], m[2], m[3]};
        *reinterpret_cast<f32x4*>(&qs[hh * T + i][lane * 8 + 4]) = (f32x4){m[4], m[5], m[6], m[7]};
      }
    }
    for (int kt = kb0; kt < k_end; kt += 32) {
      const int nkt = min(32, k_end - kt);
      __syncthreads();  // qs complete; the previous key tile is done being read
      for (int e = wave; e < 32; e += 4) {
        float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (e < nkt) {
          const int r0 = (kt + e) * block;
          wave_block_mean<D>(kunit + (int64_t)r0 * D, min(block, N - r0), lane, m);
        }
        if (lane < CH) {
          *reinterpret_cast<f32x4*>(&ks[e][lane * 8]) = (f32x4){m[0], m[1], m[2], m[3]};
          *reinterpret_cast<f32x4*>(&ks[e][lane * 8 + 4]) = (f32x4){m[4], m[5], m[6], m[7]};
        }
      }
      __syncthreads();
      for (int qt = 0; qt < nq; qt += 32) {
        const int i_hi = qb0 + min(qt + 32, nq) - 1;
        if (i_hi < kt) continue;  // wholly above the diagonal (filled above)
        float best[2][2];
        for (int hh = 0; hh < nh; ++hh) {
          float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll 4
          for (int dd = 0; dd < D; dd += 4) {
            const f32x4 a0 = *reinterpret_cast<const f32x4*>(&qs[hh * T + qt + ty][dd]);
            const f32x4 a1 = *reinterpret_cast<const f32x4*>(&qs[hh * T + qt + ty + 16][dd]);
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(&ks[tx][dd]);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(&ks[tx + 16][dd]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[0][0] = __builtin_fmaf(a0[e], b0[e], acc[0][0]);
              acc[0][1] = __builtin_fmaf(a0[e], b1[e], acc[0][1]);
              acc[1][0] = __builtin_fmaf(a1[e], b0[e], acc[1][0]);
              acc[1][1] = __builtin_fmaf(a1[e], b1[e], acc[1][1]);
            }
          }
#pragma unroll
          for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const float sc = acc[r][c] * scale;
              best[r][c] = (hh == 0) ? sc : fmaxf(best[r][c], sc);
            }
        }
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int ii = qt + ty + 16 * r, j = kt + tx + 16 * c;
            if (ii < nq && j < k_end) {
              const int i = qb0 + ii;
              float* dst = out + (int64_t)i * nB + j;
              // an earlier head chunk wrote this element (same thread)
              const float prev = hc > 0 ? *dst : NEG_INF;
              *dst = (j <= i) ? (hc > 0 ? fmaxf(prev, best[r][c]) : best[r][c]) : NEG_INF;
            }
          }
      }
    }
  }
}

template <int D, int HC>
static hipError_t launch_pooled_scores_hc(const uint16_t* q, const uint16_t* k, float* scores, int B, int Hq, int Hkv,
                                          int N, int block, int nB, float scale, hipStream_t stream) {
  // strips as long as the LDS allows (256 rows of means), shortened while the
  // grid would leave most CUs idle
  int T = 256 / HC;
  auto n_wg = [&](int t) {
    const int64_t s = (nB + t - 1) / t;
    return (int64_t)B * Hkv * (s * (s + 1) / 2);
  };
  while (T > 32 && n_wg(T) < 512) T /= 2;
  const int n_strips = (nB + T - 1) / T;
  const int64_t wgs = n_wg(T);
  if (wgs == 0) return hipSuccess;
  hipLaunchKernelGGL((pooled_scores_kernel<D, HC>), dim3((uint32_t)wgs), dim3(256), 0, stream, q, k, scores, Hq, Hkv,
                     N, block, nB, T, n_strips, scale);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_pooled_scores_d(const uint16_t* q, const uint16_t* k, float* scores, int B, int Hq, int Hkv,
                                         int N, int block, int nB, float scale, hipStream_t stream) {
  const int G = Hq / Hkv;
  if (G >= 8) return launch_pooled_scores_hc<D, 8>(q, k, scores, B, Hq, Hkv, N, block, nB, scale, stream);
  if (G >= 4) return launch_pooled_scores_hc<D, 4>(q, k, scores, B, Hq, Hkv, N, block, nB, scale, stream);
  if (G >= 2) return launch_pooled_scores_hc<D, 2>(q, k, scores, B, Hq, Hkv, N, block, nB, scale, stream);
  return launch_pooled_scores_hc<D, 1>(q, k, scores, B, Hq, Hkv, N, block, nB, scale, stream);
}

hipError_t launch_pooled_scores(const uint16_t* q, const uint16_t* k, float* scores, int B, int Hq, int Hkv, int N,
                                int d, int block, float scale, hipStream_t stream) {
  const int nB = (N + block - 1) / block;
  if (d == 64) return launch_pooled_scores_d<64>(q, k, scores, B, Hq, Hkv, N, block, nB, scale, stream);
  return launch_pooled_scores_d<128>(q, k, scores, B, Hq, Hkv, N, block, nB, scale, stream);
}

// ============================================================== top-k select
// One 64-lane wave per row (rows of up to 64 * R blocks), 4 rows per
// workgroup; the selection itself is wave_select_row (topk_row.hpp).
template <int R>
__global__ __launch_bounds__(256) void select_topk_wave_kernel(const float* __restrict__ scores,
                                                               int32_t* __restrict__ idx, int32_t* __restrict__ cnt,
                                                               int64_t n_rows, int rows_per_unit, int n_cols,
                                                               int causal, TopkParams p, int kmax) {
  __shared__ uint32_t lds_key[4][128];
  __shared__ int32_t lds_idx[4][128];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= n_rows) return;  // whole wave; no workgroup barrier below
  const int i = (int)(row % rows_per_unit);
  const int nv = causal ? i + 1 : n_cols;
  const int total = wave_select_row<R>(scores + row * (int64_t)n_cols, nv, p, idx + row * (int64_t)kmax, kmax,
                                       lds_key[wave], lds_idx[wave]);
  if ((threadIdx.x & 63) == 0 && cnt) cnt[row] = total;
}

hipError_t launch_select_topk(const float* scores, int32_t* idx, int32_t* cnt, int64_t n_rows, int rows_per_unit,
                              int n_cols, bool causal, TopkParams p, int kmax, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  const int longest = causal ? rows_per_unit : n_cols;
  const dim3 grid((uint32_t)((n_rows + 3) / 4)), block(256);
  const int c = causal ? 1 : 0;
  if (longest <= 64 * 4)
    hipLaunchKernelGGL(select_topk_wave_kernel<4>, grid, block, 0, stream, scores, idx, cnt, n_rows, rows_per_unit,
                       n_cols, c, p, kmax);
  else if (longest <= 64 * 16)
    hipLaunchKernelGGL(select_topk_wave_kernel<16>, grid, block, 0, stream, scores, idx, cnt, n_rows, rows_per_unit,
                       n_cols, c, p, kmax);
  else if (longest <= 64 * 64)
    hipLaunchKernelGGL(select_topk_wave_kernel<64>, grid, block, 0, stream, scores, idx, cnt, n_rows, rows_per_unit,
                       n_cols, c, p, kmax);
  else if (longest <= 64 * 128)  // token rows
    hipLaunchKernelGGL(select_topk_wave_kernel<128>, grid, block, 0, stream, scores, idx, cnt, n_rows, rows_per_unit,
                       n_cols, c, p, kmax);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ============================================================== marked token rows
// The general one-wave select for the causal rows whose count is -1 (rows the
// token fast path left).  Each wave scans 64 consecutive rows' counts at once
// and selects only the marked ones, so the usual (no or few marked rows)
// launch is short.
__global__ __launch_bounds__(256) void select_marked_kernel(const float* __restrict__ scores, int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ cnt, int64_t n_rows, int N,
                                                            TopkParams p, int kmax) {
  __shared__ uint32_t lds_key[4][128];
  __shared__ int32_t lds_idx[4][128];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * 64;
  if (row0 >= n_rows) return;  // whole wave
  const bool marked = row0 + lane < n_rows && cnt[row0 + lane] < 0;
  uint64_t todo = __builtin_amdgcn_ballot_w64(marked);
  while (todo) {
    const int l = __builtin_ctzll(todo);
    todo &= todo - 1;
    const int64_t row = row0 + l;
    const int nv = (int)(row % N) + 1;
    const int total = wave_select_row<128>(scores + row * (int64_t)N, nv, p, idx + row * (int64_t)kmax, kmax,
                                           lds_key[wave], lds_idx[wave]);
    if (lane == 0) cnt[row] = total;
  }
}

hipError_t launch_select_marked(const float* scores, int32_t* idx, int32_t* cnt, int64_t n_rows, int N, TopkParams p,
                                int kmax, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  const int64_t waves = (n_rows + 63) / 64;
  hipLaunchKernelGGL(select_marked_kernel, dim3((uint32_t)((waves + 3) / 4)), dim3(256), 0, stream, scores, idx, cnt,
                     n_rows, N, p, kmax);
  return hipGetLastError();
}

// ============================================================== bitmap
// One wave per row: the row's kept block ids (idx[row, 0 .. n - 1], n = cnt[row]
// or kmax) set bit j % 32 of word j / 32 in an LDS copy of the row's words
// (LDS atomic OR), which is then stored whole.  Ids outside [0, n_cols) are
// skipped.
__global__ __launch_bounds__(256) void bitmap_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
                                                     uint32_t* __restrict__ out, int64_t n_rows, int kmax, int n_cols) {
  __shared__ uint32_t words[4][DSA_MAX_BLOCKS / 32];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= n_rows) return;  // whole wave; no workgroup barrier below
  const int W = (n_cols + 31) / 32;
  for (int w = lane; w < W; w += 64) words[wave][w] = 0u;
  wave_lds_sync();
  const int n = cnt ? min(max(cnt[row], 0), kmax) : kmax;
  for (int e = lane; e < n; e += 64) {
    const int j = idx[row * kmax + e];
    if (j >= 0 && j < n_cols) atomicOr(&words[wave][j >> 5], 1u << (j & 31));
  }
  wave_lds_sync();
  for (int w = lane; w < W; w += 64) out[row * W + w] = words[wave][w];
}

hipError_t launch_bitmap(const int32_t* idx, const int32_t* cnt, uint32_t* out, int64_t n_rows, int kmax, int n_cols,
                         hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(bitmap_kernel, dim3((uint32_t)((n_rows + 3) / 4)), dim3(256), 0, stream, idx, cnt, out, n_rows,
                     kmax, n_cols);
  return hipGetLastError();
}

}  // namespace dsa
