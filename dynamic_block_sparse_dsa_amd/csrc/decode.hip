// Single-token decode over a block-sparse KV cache.
//
// Method sources (by page and section):
//   "dynamic sparse attention explainer" (zblog.xzdbk.com/559.html),
//     "动态开销与计算收益的权衡": compute the index data when the cache is
//     written rather than reselecting from raw keys every step (the fp32 block
//     means of the key cache are built once, by dsa_kv_block_means);
//     "前沿方向": GQA/MQA share the KV cache and so one selection per group;
//     "基于Top-k选择的局部-全局混合": keep the best blocks plus anchors.
//   "稀疏注意力 vs Flash Attention v2" (pnsm.cn/news/1249548.html), section 1:
//     softmax of the scaled logits over the kept keys, times V.
//
// A step is bound by HBM bandwidth: it must read the block means of the whole
// key cache and the kept K/V blocks, each once, with non-temporal loads.
//
// Scoring + selection (score_and_select): one 512-thread workgroup per
// (sequence, KV head) unit streams the unit's fp32 block means with 16-byte
// loads (d/8 lanes per block row; each wave scores one contiguous eighth of
// the blocks, batch by batch with the next batch in flight; row dot products
// reduced with DPP), scores each block by the max over the group's heads of
// q_h . kbar_j / sqrt(d) into LDS, then selects on the LDS scores -- no
// score round trip: a plain top-k keeping at most 64 candidates runs in two
// wave-level rounds (each wave keeps the best of its own eighth as soon as it
// has scored it, then one wave the best of those lists: topk_round1 and
// topk_round2), larger ones a workgroup digit-wise histogram search
// (block_select_topk); one wave runs the threshold and entropy variants
// (wave_select_row).
//
// Attention over the kept blocks works in 32-key chunks (WaveAttn): a wave
// issues all K and V loads of a chunk together, then Q K^T on
// v_mfma_f32_16x16x32_bf16 (key rows as the A operand, the group's heads as B
// columns) and P V as fp32 VALU over 16-byte V rows, with an online softmax.
//
// Two ways to run a step:
//   * fused (>= 256 units, one per CU): decode_fused_kernel -- the unit's
//     workgroup selects, then its 8 waves walk the unit's chunks (first come
//     first served, or in a fixed round-robin order under DSA_DETERMINISTIC)
//     and merge through LDS into o and lse.  One launch, no workspace.
//   * split (fewer units): decode_select_kernel writes idx; decode_attn_kernel
//     runs split-K over the kept blocks (one 256-thread workgroup per (unit,
//     split)) and writes a partial (max, sum, acc[d]) per head;
//     decode_combine_kernel merges the partials.
#include <mutex>

#include "decode_common.hpp"
#include "topk_row.hpp"

namespace dsa {

#define CONST_AS __attribute__((address_space(4)))

// ============================================================== 1. score + select
// Score every block of one (sequence, KV head) unit into LDS and select its
// kept blocks (written ascending to out, -1 padded to kmax; out may be
// global or LDS).  All NT = 512 threads of the workgroup take part.  Scores:
// block l * R + e at sc[e * 64 + l].  Wave w scores the blocks
// w B .. w B + B - 1 (B = 64 R / 8), batch by batch with the next batch in
// flight, and a plain top-k row keeping at most 64 candidates then runs its
// first selection round on them at once (topk_round1: the wave's best m), so
// waves that finish scoring early select while others still load.
// pre_select() runs in every thread once every wave is done, before the
// second round (a caller's prefetch stays in flight through it).  The
// selection is complete only after the caller's next barrier.
template <int D, int G, int R, typename Pre>
__device__ __forceinline__ void score_and_select(const DecodeArgs& a, const TopkParams& p, int unit, float* sc,
                                                 uint32_t* lds_key, int32_t* lds_idx, uint32_t* bsel,
                                                 int32_t* out, Pre&& pre_select) {
  constexpr int NT = 512, NW = NT / 64;
  constexpr int TPR = D / 8;       // lanes per block row (8 floats each)
  constexpr int WROWS = 64 / TPR;  // rows per wave per pass
  constexpr int UNR = 8;           // passes per batch
  constexpr int BR = WROWS * UNR;  // rows per batch (16 KiB of fp32 means at d = 128)
  constexpr int BPW = 64 * R / NW;  // blocks per wave
  static_assert(BPW % BR == 0, "whole batches per wave");
  const int64_t s = unit / a.Hkv;
  const int g = unit % a.Hkv;
  const int t = threadIdx.x, lane = t & 63, c = lane % TPR, rl = lane / TPR;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int nB = a.nB;
  const int nbatch = (nB + BR - 1) / BR;

  float qv[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) load_q_halves<D>(a.q + (s * a.Hq + g * G + hh) * (int64_t)D, c, qv[hh]);
  // rows past the end are clamped (loaded again, never stored)
  const float* kb = a.kbar + (int64_t)unit * nB * D + 4 * c;
  auto load = [&](f32x4(&kv)[UNR][2], int b) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int row = min(b * BR + u * WROWS + rl, nB - 1);
      kv[u][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kb + (int64_t)row * D));
      kv[u][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kb + (int64_t)row * D + D / 2));
    }
  };
  auto score = [&](const f32x4(&kv)[UNR][2], int b) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float best = -__builtin_inff();
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          part = __builtin_fmaf(qv[hh][e], kv[u][0][e], part);
          part = __builtin_fmaf(qv[hh][4 + e], kv[u][1][e], part);
        }
        best = fmaxf(best, group_sum<TPR>(part) * a.scale);
      }
      const int row = b * BR + u * WROWS + rl;
      if (c == 0 && row < nB) sc[(row % R) * 64 + row / R] = best;
    }
  };
  const int b_lo = wave * (BPW / BR), b_hi = min(b_lo + BPW / BR, nbatch);
  f32x4 k0[UNR][2], k1[UNR][2];
  if (b_lo < b_hi) load(k0, b_lo);
  for (int b = b_lo; b < b_hi; b += 2) {
    if (b + 1 < b_hi) load(k1, b + 1);
    score(k0, b);
    if (b + 1 >= b_hi) break;
    if (b + 2 < b_hi) load(k0, b + 2);
    score(k1, b + 1);
  }
  const TopkRow tr(nB, p);
  const bool two = p.mode == DSA_SELECT_TOPK && tr.two_round(nB);
  const int ls = tr.m <= 32 ? 32 : 64;
  uint32_t* scratch2 = bsel + BSEL_SCRATCH_WORDS;
  if (two) {
    wave_lds_sync();  // the wave's own scores
    topk_round1<R, NW>(sc, tr, ls, scratch2);
  }
  __syncthreads();
  pre_select();
  if (two) {
    if (wave == 0) {
      if (ls == 32) topk_round2<NW, NW / 2>(tr, nB, out, a.kmax, ls, scratch2);
      else topk_round2<NW, NW>(tr, nB, out, a.kmax, ls, scratch2);
    }
  } else if (p.mode == DSA_SELECT_TOPK) {
    block_select_topk<R, NT>(sc, nB, p, out, a.kmax, bsel);  // the workgroup selects
  } else if (t < 64) {
    wave_select_row<R, true>(sc, nB, p, out, a.kmax, lds_key, lds_idx);  // one wave selects
  }
}

template <int D, int G, int R>
__global__ __launch_bounds__(512) void decode_select_kernel(DecodeArgs a, TopkParams p) {
  __shared__ float sc[64 * R];
  __shared__ uint32_t lds_key[128];
  __shared__ int32_t lds_idx[128];
  __shared__ uint32_t bsel[BSEL_SCRATCH_WORDS + BSEL2_SCRATCH_WORDS];
  score_and_select<D, G, R>(a, p, blockIdx.x, sc, lds_key, lds_idx, bsel, a.idx + (int64_t)blockIdx.x * a.kmax,
                            [] {});
}

// ============================================================== 2. attention
// ------------------------------------------------------------ split path
// Split-K over the kept blocks, one 256-thread workgroup per (unit, split),
// one chunk per wave at a time; the workgroup writes a partial per head (the
// split count: decode_splits, plan.cpp).

// Library-owned scratch for dsa_decode_noalloc (callers that cannot allocate):
// the split partials [S * Hkv, nsplit, G, d + 2] fp32 of any shape the split
// path takes fit in it (S * Hkv < 256 units, nsplit <= ceil(1024 / units):
// under 1 280 (unit, split) pairs x 8 heads x 130 floats = 5.3 MB).  One copy
// per GPU, held until the process ends.  Host code never uses the array's
// name as an address: decode_noalloc_scratch() looks the device address up
// once per device and passes that pointer to the kernels.
static __device__ __align__(256) unsigned char scratch[DSA_DECODE_NOALLOC_MAX_BYTES];

hipError_t decode_noalloc_scratch(void** out) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* ptr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

template <int D, int BLK, int G>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeArgs a) {
  using C = DecCfg<D, G>;
  constexpr int WAVES = 4;
  constexpr int CPB = BLK / C::CK;         // chunks per block
  __shared__ __align__(1024) uint16_t vtile[WAVES][C::CK * D];  // V rows of the wave's current chunk
  __shared__ float mw[WAVES][G], lw[WAVES][G];
  __shared__ float accw[WAVES][G][D];

  const int unit = blockIdx.x / a.nsplit;
  const int split = blockIdx.x % a.nsplit;
  const int bps = (a.kmax + a.nsplit - 1) / a.nsplit;
  const int t0 = split * bps, t1 = min(a.kmax, t0 + bps);
  const int64_t s = unit / a.Hkv;
  const int g = unit % a.Hkv;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = a.L;
  const uint16_t* kb = a.kc + (int64_t)unit * L * D;
  const uint16_t* vb = a.vc + (int64_t)unit * L * D;
  const CONST_AS int32_t* irow = (const CONST_AS int32_t*)(a.idx + (int64_t)unit * a.kmax);
  const float NEG_INF = -__builtin_inff();

  WaveAttn<D, G> wa;
  wa.init(a, s, g);
  ChunkRegs<D, G> r;
  for (int ch = t0 * CPB + wave; ch < t1 * CPB; ch += WAVES) {
    const int blk = irow[ch / CPB];
    if (blk < 0) continue;  // padding (a shorter row): nothing to attend
    const int key0 = blk * BLK + (ch % CPB) * C::CK;
    if (key0 >= L) continue;  // a chunk past the end of a ragged last block
    wa.load(r, kb, vb, key0, L);
    wa.step(r, key0, L, a.scale_log2, (LDS_AS uint16_t*)vtile[wave]);
  }
  wa.to_lds(mw[wave], lw[wave], accw[wave]);
  __syncthreads();
  for (int e = tid; e < G * (D + 2); e += 256) {
    const int hh = e / (D + 2), c = e % (D + 2);
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, mw[w][hh]);
    float v = 0.f;
    if (c == 0) {
      v = M;  // -inf: the split attended nothing, and the combine skips it
    } else if (M != NEG_INF) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        const float f = __builtin_amdgcn_exp2f(mw[w][hh] - M);  // 0 for a wave with no chunk
        v += f * (c == 1 ? lw[w][hh] : accw[w][hh][c - 2]);
      }
    }
    a.partial[(((int64_t)unit * a.nsplit + split) * G + hh) * (D + 2) + c] = v;
  }
}

// One thread per (unit, head, dim); the split maxima are read first, then the
// sums and accumulators, all loads independent.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ partial,
                                                             uint16_t* __restrict__ o, float* __restrict__ lse,
                                                             int Hq, int Hkv, int nsplit, int64_t n_items) {
  const int G = Hq / Hkv;
  const int64_t item = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (unit, hh, dd)
  if (item >= n_items) return;
  const int dd = (int)(item % D);
  const int64_t uh = item / D;
  const int hh = (int)(uh % G);
  const int64_t unit = uh / G;
  const float* p = partial + (unit * nsplit * G + hh) * (D + 2);
  const int stride = G * (D + 2);
  float mv[DEC_MAX_SPLITS];
  float M = -__builtin_inff();
#pragma unroll
  for (int c = 0; c < DEC_MAX_SPLITS; ++c) {
    mv[c] = (c < nsplit) ? p[c * stride] : -__builtin_inff();
    M = fmaxf(M, mv[c]);
  }
  float l = 0.f, v = 0.f;
#pragma unroll
  for (int c = 0; c < DEC_MAX_SPLITS; ++c) {
    if (c < nsplit && mv[c] != -__builtin_inff()) {
      const float f = __builtin_amdgcn_exp2f(mv[c] - M);
      l += f * p[c * stride + 1];
      v += f * p[c * stride + 2 + dd];
    }
  }
  const int64_t s = unit / Hkv;
  const int g = (int)(unit % Hkv);
  const int64_t oh = s * Hq + g * G + hh;
  o[oh * D + dd] = (uint16_t)f32_to_bf16_rne(v / l);
  if (lse && dd == 0) lse[oh] = (M + __log2f(l)) * 0.69314718055994531f;
}

// ------------------------------------------------------------ fused path
// One 512-thread workgroup per unit does the whole step: score + select as
// above (the selection goes to LDS and to idx), then its 8 waves walk the
// unit's chunks (taken from an LDS counter, or round-robin under
// DSA_DETERMINISTIC; two chunks in flight per wave) and merge through LDS
// straight into o and lse.  No workspace, one launch.  Used
// when there are enough units to give every CU one.
template <int D, int BLK, int G, int R>
__global__ __launch_bounds__(512) void decode_fused_kernel(DecodeArgs a, TopkParams p) {
  using C = DecCfg<D, G>;
  constexpr int NW = 8;
  constexpr int CPB = BLK / C::CK;
  __shared__ float sc[64 * R];
  __shared__ uint32_t lds_key[128];
  __shared__ int32_t lds_idx[128];
  __shared__ uint32_t bsel[BSEL_SCRATCH_WORDS + BSEL2_SCRATCH_WORDS];
  __shared__ int next_batch;
  __shared__ int32_t sel[64 * R];          // kept blocks (kmax <= nB <= 64 R)
  __shared__ __align__(1024) uint16_t vtile[NW][C::CK * D];
  __shared__ float mw[NW][G], lw[NW][G];
  __shared__ float accw[NW][G][D];
  const int unit = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t s = unit / a.Hkv;
  const int g = unit % a.Hkv;
  const int L = a.L;
  const float NEG_INF = -__builtin_inff();

  const int kmax = a.kmax;  // every unit keeps exactly kmax blocks (all see nB)
  const int nch = kmax * CPB;
  const int nB = a.nB;
  // With the sink and the last block forced (and distinct) their chunks are
  // known before the selection: they are taken first (logical chunks
  // 0 .. 2 CPB - 1), so waves 1 .. 2 CPB - 1 issue their loads before the
  // selection runs.  Logical chunk j -> chunk of the ascending selection.
  const bool early = (p.flags & 3u) == 3u && nB >= 2 && kmax >= 2;
  auto phys = [&](int j) {
    if (!early || j < CPB) return j;
    return j < 2 * CPB ? nch - 2 * CPB + j : j - CPB;
  };
  auto forced_key = [&](int j) {  // j < 2 CPB, early only
    const int key0 = j < CPB ? j * C::CK : (nB - 1) * BLK + (j - CPB) * C::CK;
    return key0 < L ? key0 : -1;
  };
  // chunk i: part i % CPB of kept block i / CPB; -1 for padding, or past the
  // end of a ragged last block
  auto key_of = [&](int j) {
    if (j >= nch) return -1;
    const int i = phys(j);
    const int blk = sel[i / CPB];
    const int key0 = blk * BLK + (i % CPB) * C::CK;
    return (blk >= 0 && key0 < L) ? key0 : -1;
  };
  const uint16_t* kb = a.kc + (int64_t)unit * L * D;
  const uint16_t* vb = a.vc + (int64_t)unit * L * D;
  WaveAttn<D, G> wa;
  ChunkRegs<D, G> rA, rB;

  const bool pre = early && wave >= 1 && wave < 2 * CPB && wave < NW;
  int kA = -1;
  score_and_select<D, G, R>(a, p, unit, sc, lds_key, lds_idx, bsel, sel, [&] {
    wa.init(a, s, g);  // lane mapping + q; every later load depends on it
    if (pre) {
      kA = forced_key(wave);
      if (kA >= 0) wa.load(rA, kb, vb, kA, L);
    }
  });
  // LDS-only barriers from here to the walk, so the preloads stay in flight
  lds_barrier();
  for (int e = tid; e < kmax; e += 512) a.idx[(int64_t)unit * kmax + e] = sel[e];
  if (tid == 0) next_batch = NW;
  lds_barrier();
  // chunks 0 .. NW-1 go to the waves in order, then each wave takes the next
  // free chunk from an LDS counter (next_batch is free again: the selection
  // barrier is behind us), keeping one more chunk in flight than it computes.
  // DSA_DETERMINISTIC: wave w takes chunks w, w + NW, w + 2 NW, ... instead,
  // so the merge below adds the same partials in the same order on every call
  // (first come first served balances the waves a little better).
  const bool fixed = (p.flags & DSA_DETERMINISTIC) != 0u;
  int next_chunk = wave + NW;
  auto grab = [&]() {
    if (fixed) {
      const int v = next_chunk;
      next_chunk += NW;
      return v;
    }
    int v = 0;
    if ((tid & 63) == 0) v = atomicAdd(&next_batch, 1);
    return __builtin_amdgcn_readfirstlane(__shfl(v, 0, 64));
  };
  int iA = wave;
  if (!pre) {
    kA = key_of(iA);
    if (kA >= 0) wa.load(rA, kb, vb, kA, L);
  }
  int iB = grab();
  while (iA < nch) {
    const int kB = key_of(iB);
    if (kB >= 0) wa.load(rB, kb, vb, kB, L);
    if (kA >= 0) wa.step(rA, kA, L, a.scale_log2, (LDS_AS uint16_t*)vtile[wave]);
    if (iB >= nch) break;
    iA = grab();
    kA = key_of(iA);
    if (kA >= 0) wa.load(rA, kb, vb, kA, L);
    if (kB >= 0) wa.step(rB, kB, L, a.scale_log2, (LDS_AS uint16_t*)vtile[wave]);
    iB = grab();
  }
  wa.to_lds(mw[wave], lw[wave], accw[wave]);
  __syncthreads();
  for (int e = tid; e < G * D; e += 512) {
    const int hh = e / D, dd = e % D;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mw[w][hh]);
    float l = 0.f, v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(mw[w][hh] - M);  // 0 for a wave with no chunk
      l += f * lw[w][hh];
      v += f * accw[w][hh][dd];
    }
    const int64_t oh = s * a.Hq + g * G + hh;
    a.o[oh * D + dd] = (uint16_t)f32_to_bf16_rne(v / l);
    if (a.lse && dd == 0) a.lse[oh] = (M + __log2f(l)) * 0.69314718055994531f;
  }
}

// ============================================================== launch
template <int D, int G>
static void launch_select(const DecodeArgs& a, TopkParams p, hipStream_t stream) {
  const dim3 grid((uint32_t)((int64_t)a.S * a.Hkv)), blk(512);
  if (a.nB <= 64 * 16)
    hipLaunchKernelGGL((decode_select_kernel<D, G, 16>), grid, blk, 0, stream, a, p);
  else
    hipLaunchKernelGGL((decode_select_kernel<D, G, 64>), grid, blk, 0, stream, a, p);
}

template <int D, int BLK, int G>
static void launch_fused(const DecodeArgs& a, TopkParams p, hipStream_t stream) {
  const dim3 grid((uint32_t)((int64_t)a.S * a.Hkv)), blk(512);
  if (a.nB <= 64 * 16)
    hipLaunchKernelGGL((decode_fused_kernel<D, BLK, G, 16>), grid, blk, 0, stream, a, p);
  else
    hipLaunchKernelGGL((decode_fused_kernel<D, BLK, G, 64>), grid, blk, 0, stream, a, p);
}

template <int D, int BLK>
static hipError_t launch_decode_d(const DecodeArgs& a, TopkParams p, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return hipErrorInvalidValue;
  if ((int64_t)a.S * a.Hkv >= DEC_FUSED_MIN_UNITS) {
    switch (G) {
      case 1: launch_fused<D, BLK, 1>(a, p, stream); break;
      case 2: launch_fused<D, BLK, 2>(a, p, stream); break;
      case 4: launch_fused<D, BLK, 4>(a, p, stream); break;
      case 8: launch_fused<D, BLK, 8>(a, p, stream); break;
    }
    return hipGetLastError();
  }
  const dim3 grid((uint32_t)((int64_t)a.S * a.Hkv * a.nsplit)), blk(256);
  switch (G) {
    case 1: launch_select<D, 1>(a, p, stream); break;
    case 2: launch_select<D, 2>(a, p, stream); break;
    case 4: launch_select<D, 4>(a, p, stream); break;
    case 8: launch_select<D, 8>(a, p, stream); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_attn_kernel<D, BLK, 1>), grid, blk, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_attn_kernel<D, BLK, 2>), grid, blk, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_attn_kernel<D, BLK, 4>), grid, blk, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_attn_kernel<D, BLK, 8>), grid, blk, 0, stream, a); break;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items = (int64_t)a.S * a.Hq * D;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((uint32_t)((items + 255) / 256)), dim3(256), 0, stream,
                     a.partial, a.o, a.lse, a.Hq, a.Hkv, a.nsplit, items);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int d, TopkParams p, hipStream_t stream) {
  if ((int64_t)a.S * a.Hkv == 0) return hipSuccess;
  if (d == 64) return a.block == 64 ? launch_decode_d<64, 64>(a, p, stream) : launch_decode_d<64, 128>(a, p, stream);
  return a.block == 64 ? launch_decode_d<128, 64>(a, p, stream) : launch_decode_d<128, 128>(a, p, stream);
}

}  // namespace dsa
