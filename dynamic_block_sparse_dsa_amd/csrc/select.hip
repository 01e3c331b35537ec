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
// One workgroup per (unit, block): 256 threads read the block's rows as
// 16-byte chunks (D/8 chunks per row, 256/(D/8) row groups), sum them in fp32,
// reduce the row groups through LDS and divide by the number of real rows.
// Two tensors in one launch: the first n0 units of x0, then those of x1.
template <int D>
__global__ __launch_bounds__(256) void block_means_kernel(const uint16_t* __restrict__ x0, float* __restrict__ xbar0,
                                                          int64_t n0, const uint16_t* __restrict__ x1,
                                                          float* __restrict__ xbar1, int N, int block, int nB) {
  constexpr int CH = D / 8;        // 16-byte chunks per row
  constexpr int RG = 256 / CH;     // row groups
  __shared__ float part[RG][D + 1];
  int64_t wg = blockIdx.x;
  const uint16_t* x = x0;
  float* xbar = xbar0;
  if (wg >= n0 * nB) {
    wg -= n0 * nB;
    x = x1;
    xbar = xbar1;
  }
  const int64_t unit = wg / nB;
  const int j = (int)(wg % nB);
  const int t = threadIdx.x, c = t % CH, rg = t / CH;
  const int r0 = j * block;
  const int rows = min(block, N - r0);
  const uint16_t* base = x + (unit * N + r0) * (int64_t)D + c * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = rg; r < rows; r += RG) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(base + (int64_t)r * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_lo(w[e]);
      acc[2 * e + 1] += bf16_hi(w[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rg][c * 8 + e] = acc[e];
  __syncthreads();
  if (t < D) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) s += part[g][t];
    xbar[(unit * nB + j) * (int64_t)D + t] = s / (float)rows;
  }
}

hipError_t launch_block_means2(const uint16_t* x0, float* xbar0, int64_t n0, const uint16_t* x1, float* xbar1,
                               int64_t n1, int N, int d, int block, hipStream_t stream) {
  const int nB = (N + block - 1) / block;
  const int64_t n_wg = (n0 + n1) * nB;
  if (n_wg == 0) return hipSuccess;
  if (d == 64)
    hipLaunchKernelGGL(block_means_kernel<64>, dim3((uint32_t)n_wg), dim3(256), 0, stream, x0, xbar0, n0, x1, xbar1,
                       N, block, nB);
  else
    hipLaunchKernelGGL(block_means_kernel<128>, dim3((uint32_t)n_wg), dim3(256), 0, stream, x0, xbar0, n0, x1, xbar1,
                       N, block, nB);
  return hipGetLastError();
}

hipError_t launch_block_means(const uint16_t* x, float* xbar, int64_t n_units, int N, int d, int block,
                              hipStream_t stream) {
  return launch_block_means2(x, xbar, n_units, nullptr, nullptr, 0, N, d, block, stream);
}

// ============================================================== block scores
// One 256-thread workgroup per 32x32 tile of the score matrix of one (batch,
// KV head): thread (ty, tx) owns rows ty, ty+16 and columns tx, tx+16.  Both
// tiles of means are staged whole in LDS (row pitch D+4 floats: the float4
// reads of 16 K rows hit distinct bank groups, the Q reads are broadcasts);
// the K tile and the first Q tile are fetched together; every head of the
// group is scored against the K tile and the max is kept.  Tiles strictly
// above the diagonal are -inf.
template <int D>
__global__ __launch_bounds__(256) void block_scores_kernel(const float* __restrict__ qbar,
                                                           const float* __restrict__ kbar, float* __restrict__ scores,
                                                           int Hq, int Hkv, int nB, float scale, int n_tiles) {
  constexpr int PITCH = D + 4;  // rows 16-byte aligned, one bank group apart: conflict-free float4 reads
  constexpr int PER_T = 32 * D / 4 / 256;  // float4 pieces of a tile per thread
  __shared__ __align__(16) float qs[32][PITCH];
  __shared__ __align__(16) float ks[32][PITCH];
  const int per_unit = n_tiles * n_tiles;
  const int64_t unit = blockIdx.x / per_unit;  // b * Hkv + g
  const int tile = blockIdx.x % per_unit;
  const int ti = tile / n_tiles, tj = tile % n_tiles;
  const int t = threadIdx.x, tx = t % 16, ty = t / 16;
  const int i0 = ti * 32, j0 = tj * 32;
  float* out = scores + unit * (int64_t)nB * nB;
  const float NEG_INF = -__builtin_inff();
  if (tj > ti) {
    for (int e = t; e < 32 * 32; e += 256) {
      const int i = i0 + e / 32, j = j0 + e % 32;
      if (i < nB && j < nB) out[(int64_t)i * nB + j] = NEG_INF;
    }
    return;
  }
  const int G = Hq / Hkv;
  const int64_t b = unit / Hkv, g = unit % Hkv;
  const float* kb = kbar + unit * (int64_t)nB * D;
  // a 32-row tile of means: global -> registers (rows past nB read as 0), then LDS
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
  float best[2][2];
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
    float acc[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll 4
    for (int dd = 0; dd < D; dd += 4) {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(&qs[ty][dd]);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(&qs[ty + 16][dd]);
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
      const int i = i0 + ty + 16 * r, j = j0 + tx + 16 * c;
      if (i < nB && j < nB) out[(int64_t)i * nB + j] = (j <= i) ? best[r][c] : NEG_INF;
    }
}

hipError_t launch_block_scores(const float* qbar, const float* kbar, float* scores, int B, int Hq, int Hkv, int nB,
                               int d, float scale, hipStream_t stream) {
  const int n_tiles = (nB + 31) / 32;
  const int64_t n_wg = (int64_t)B * Hkv * n_tiles * n_tiles;
  if (n_wg == 0) return hipSuccess;
  if (d == 64)
    hipLaunchKernelGGL(block_scores_kernel<64>, dim3((uint32_t)n_wg), dim3(256), 0, stream, qbar, kbar, scores, Hq,
                       Hkv, nB, scale, n_tiles);
  else
    hipLaunchKernelGGL(block_scores_kernel<128>, dim3((uint32_t)n_wg), dim3(256), 0, stream, qbar, kbar, scores, Hq,
                       Hkv, nB, scale, n_tiles);
  return hipGetLastError();
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
