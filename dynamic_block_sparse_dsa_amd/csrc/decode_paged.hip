// Decode over a paged KV cache with a length per sequence, and the cache-side
// work that keeps its index data current (token appends, per-page block means).
//
// Method sources: "dynamic sparse attention explainer" (zblog.xzdbk.com/559.html),
//   "动态开销与计算收益的权衡": build the index data when the cache is written
//   (here: each page's key block mean, recomputed when a token lands in it);
//   "硬件友好的稀疏计算实现": tie the block decision to the KV cache's blocks
//   (here a page is one block); "基于Top-k选择的局部-全局混合": the best blocks
//   plus anchors and a local window.  "稀疏注意力 vs Flash Attention v2"
//   (pnsm.cn/news/1249548.html), section 1: softmax of the scaled logits over
//   the kept keys, times V.
//
// Layout: pools [n_pages, Hkv, BLK, D] bf16 (one (page, head) tile is one
// contiguous BLK * D * 2-byte run), block means [n_pages, Hkv, D] fp32,
// block table [S, max_blocks] int32 (page of each logical block), lengths [S].
//
// decode_paged_kernel: one 512-thread workgroup per (sequence, KV head) unit.
//   The unit's nB = ceil(L / BLK) block means are read through the block table
//   (16-byte non-temporal loads, d/8 lanes per row, wave w scoring its own
//   range of blocks) and scored by the max over the group's heads of
//   q . kbar / sqrt(d) into LDS; each wave runs the first round of a top-k
//   selection on its range as soon as it is scored, then one wave the second
//   (the whole workgroup, or one wave, for rows the two rounds do not cover
//   and for the threshold and entropy variants).  Meanwhile the waves whose
//   first chunk lies in a forced block (sink, last block) load it.  The 8
//   waves then walk the kept blocks' 32-key chunks with WaveAttn (page base
//   from the table, keys past the sequence's end masked), taking chunks first
//   come first served, or w, w + 8, ... under DSA_DETERMINISTIC so that every
//   call merges the same partials in the same order, and merge through LDS
//   into o and lse.
// kv_append_kernel: one workgroup per sequence: writes the new token's K and V
//   rows into slot L % BLK of page table[L / BLK] for every KV head, recomputes
//   that page's key mean over its rows 0 .. L % BLK, then advances the length.
// paged_means_kernel: one wave per (sequence, logical block, KV head): the
//   mean of the page's rows below the sequence's length.
#include <type_traits>

#include "decode_common.hpp"
#include "topk_row.hpp"

namespace dsa {

template <int D, int BLK, int G, int R, bool F8>
__global__ __launch_bounds__(512) void decode_paged_kernel(PagedArgs a, TopkParams p) {
  using C = DecCfg<D, G>;
  constexpr int NT = 512, NW = 8;
  constexpr int CPB = BLK / C::CK;
  constexpr int TPR = D / 8, WROWS = 64 / TPR, UNR = 8, BR = WROWS * UNR;
  __shared__ float sc[64 * R];
  __shared__ uint32_t lds_key[128];
  __shared__ int32_t lds_idx[128];
  __shared__ uint32_t bsel[BSEL_SCRATCH_WORDS + BSEL2_SCRATCH_WORDS];
  __shared__ int next_batch, n_sel;
  __shared__ int32_t sel[64 * R];
  __shared__ int32_t psel[64 * R];  // pages: of the scanned rows, then of the kept blocks
  __shared__ __align__(1024) uint16_t vtile[NW][C::CK * D];
  __shared__ float mw[NW][G], lw[NW][G];
  __shared__ float accw[NW][G][D];
  const int unit = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t s = unit / a.Hkv;
  const int g = unit % a.Hkv;
  const int L = min(max(a.lengths[s], 0), a.max_blocks * BLK);
  const int nB = (L + BLK - 1) / BLK;
  const int32_t* trow = a.table + s * (int64_t)a.max_blocks;
  auto page_of = [&](int j) { return min(max(trow[j], 0), a.n_pages - 1); };
  const int kmax = a.kmax;

  if (L == 0) {  // an empty sequence: nothing kept, o = 0, lse = -inf
    for (int e = tid; e < kmax; e += NT) a.idx[(int64_t)unit * kmax + e] = -1;
    for (int e = tid; e < G * D; e += NT) a.o[((s * a.Hq + g * G) * (int64_t)D) + e] = 0;
    if (tid < G && a.lse) a.lse[s * a.Hq + g * G + tid] = -__builtin_inff();
    if (tid == 0 && a.cnt) a.cnt[unit] = 0;
    return;
  }

  // The attention's chunks: chunk i is part i % CPB of kept block i / CPB.
  // With the sink and the last block forced (and distinct) their chunks are
  // known before the selection: they are taken first (logical chunks 0 ..
  // 2 CPB - 1), so waves 1 .. 2 CPB - 1 issue their loads while wave 0 runs
  // the selection's second round.  Logical chunk j -> chunk of the ascending
  // selection (ns kept blocks, ns * CPB chunks).
  using Regs = typename std::conditional<F8, ChunkRegs8<D, G>, ChunkRegs<D, G>>::type;
  const bool early = (p.flags & 3u) == 3u && nB >= 2;
  struct Ref {
    int64_t tile;   // (page, head) tile: element offset into the pools
    int key0, lim;  // key0 < 0: nothing
  };
  auto ref_page = [&](int blk, int page, int part) {
    Ref r{0, -1, 0};
    const int key0 = part * C::CK;
    const int lim = min(BLK, L - blk * BLK);
    if (key0 >= lim) return r;
    r.tile = ((int64_t)page * a.Hkv + g) * BLK;
    r.key0 = key0;
    r.lim = lim;
    return r;
  };
  auto ref_blk = [&](int blk, int part) { return ref_page(blk, page_of(blk), part); };
  WaveAttn<D, G> wa;
  Regs rA, rB;
  auto load = [&](Regs& rr, const Ref& f) {
    if constexpr (F8)
      wa.load8(rr, a.k8 + f.tile * D, a.v8 + f.tile * D, a.ksc + f.tile, a.vsc + f.tile, f.key0, f.lim);
    else
      wa.load(rr, a.kp + f.tile * D, a.vp + f.tile * D, f.key0, f.lim);
  };
  const bool pre = early && wave >= 1 && wave < 2 * CPB && wave < NW;
  Ref fA{0, -1, 0};

  // ---- scores of the nB blocks (through the table), then the selection.
  // Wave w scores blocks w BPW .. w BPW + BPW - 1 with its next batch in
  // flight, then (a plain top-k row keeping at most 64 candidates) runs the
  // selection's first round on them at once, while other waves still load.
  {
    constexpr int BPW = 64 * R / NW;  // blocks per wave
    static_assert(BPW % BR == 0, "whole batches per wave");
    const int c = lane % TPR, rl = lane / TPR;
    const int nbatch = (nB + BR - 1) / BR;
    float qv[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) load_q_halves<D>(a.q + (s * a.Hq + g * G + hh) * (int64_t)D, c, qv[hh]);
    // the pages of the wave's own rows into LDS first (psel, free until the
    // selection), so that no table read waits behind the mean loads in flight
    for (int e = lane; e < BPW; e += 64) {
      const int row = wave * BPW + e;
      if (row < nB) psel[row] = page_of(row);
    }
    wave_lds_sync();
    auto load_means = [&](f32x4(&kv)[UNR][2], int b) {
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int row = min(b * BR + u * WROWS + rl, nB - 1);  // in the wave's range
        const float* kr = a.kbar + ((int64_t)psel[row] * a.Hkv + g) * D + 4 * c;
        kv[u][0] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kr));
        kv[u][1] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kr + D / 2));
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
    if (b_lo < b_hi) load_means(k0, b_lo);
    for (int b = b_lo; b < b_hi; b += 2) {
      if (b + 1 < b_hi) load_means(k1, b + 1);
      score(k0, b);
      if (b + 1 >= b_hi) break;
      if (b + 2 < b_hi) load_means(k0, b + 2);
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
    wa.init(a.q, a.Hq, s, g, F8);  // lane mapping + q; every later load depends on it
    if (pre) {  // forced chunk `wave`: part of block 0 or of block nB - 1
      fA = wave < CPB ? ref_blk(0, wave) : ref_blk(nB - 1, wave - CPB);
      if (fA.key0 >= 0) load(rA, fA);
    }
    if (two) {
      if (wave == 0) {
        if (ls == 32) topk_round2<NW, NW / 2>(tr, nB, sel, kmax, ls, scratch2);
        else topk_round2<NW, NW>(tr, nB, sel, kmax, ls, scratch2);
      }
      if (tid == 0) n_sel = tr.nf + tr.m;
    } else if (p.mode == DSA_SELECT_TOPK) {  // the workgroup selects
      const int n = block_select_topk<R, NT>(sc, nB, p, sel, kmax, bsel);
      if (tid == 0) n_sel = n;
    } else if (tid < 64) {  // one wave selects
      const int n = wave_select_row<R, true>(sc, nB, p, sel, kmax, lds_key, lds_idx);
      if (tid == 0) n_sel = n;
    }
    // LDS-only barriers from here to the walk, so the preloads stay in flight
    lds_barrier();
  }
  const int ns = n_sel;
  // the kept blocks' pages, looked up once (by wave 0, which has no forced-chunk
  // loads in flight to wait behind): a table read inside the walk would make
  // each new chunk wait for the loads issued before it (vmcnt is in order)
  if (wave == 0)
    for (int e = lane; e < ns; e += 64) psel[e] = page_of(sel[e]);
  for (int e = tid; e < kmax; e += NT) a.idx[(int64_t)unit * kmax + e] = sel[e];
  if (tid == 0 && a.cnt) a.cnt[unit] = ns;
  if (tid == 0) next_batch = NW;
  lds_barrier();

  // ---- attention over the kept blocks' chunks
  const int nch = ns * CPB;
  auto phys = [&](int j) {
    if (!early || j < CPB) return j;
    return j < 2 * CPB ? nch - 2 * CPB + j : j - CPB;
  };
  auto ref_of = [&](int j) {
    if (j >= nch) return Ref{0, -1, 0};
    const int i = phys(j);
    return ref_page(sel[i / CPB], psel[i / CPB], i % CPB);
  };
  // chunks 0 .. NW-1 go to the waves in order, then each wave takes the next
  // free chunk from an LDS counter (next_batch is free again), keeping one
  // more chunk in flight than it computes.  DSA_DETERMINISTIC: wave w takes
  // chunks w, w + NW, w + 2 NW, ... instead, so the merge below adds the same
  // partials in the same order on every call.
  const bool fixed = (p.flags & DSA_DETERMINISTIC) != 0u;
  int next_chunk = wave + NW;
  auto grab = [&]() {
    if (fixed) {
      const int v = next_chunk;
      next_chunk += NW;
      return v;
    }
    int v = 0;
    if (lane == 0) v = atomicAdd(&next_batch, 1);
    return __builtin_amdgcn_readfirstlane(__shfl(v, 0, 64));
  };
  int iA = wave;
  if (!pre) {
    fA = ref_of(iA);
    if (fA.key0 >= 0) load(rA, fA);
  }
  int iB = grab();
  while (iA < nch) {
    const Ref fB = ref_of(iB);
    if (fB.key0 >= 0) load(rB, fB);
    if (fA.key0 >= 0) wa.step(rA, fA.key0, fA.lim, a.scale_log2, (LDS_AS uint16_t*)vtile[wave]);
    if (iB >= nch) break;
    iA = grab();
    fA = ref_of(iA);
    if (fA.key0 >= 0) load(rA, fA);
    if (fB.key0 >= 0) wa.step(rB, fB.key0, fB.lim, a.scale_log2, (LDS_AS uint16_t*)vtile[wave]);
    iB = grab();
  }
  wa.to_lds(mw[wave], lw[wave], accw[wave]);
  __syncthreads();
  for (int e = tid; e < G * D; e += NT) {
    const int hh = e / D, dd = e % D;
    float M = -__builtin_inff();
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

// ============================================================== appends
template <int D, int BLK>
__global__ __launch_bounds__(256) void kv_append_kernel(const uint16_t* __restrict__ k_new,
                                                        const uint16_t* __restrict__ v_new,
                                                        const int32_t* __restrict__ table, int32_t* lengths,
                                                        uint16_t* __restrict__ kp, uint16_t* __restrict__ vp,
                                                        float* __restrict__ kbar, int Hkv, int max_blocks,
                                                        int n_pages) {
  const int64_t s = blockIdx.x;
  const int tid = threadIdx.x;
  const int pos = lengths[s];
  __syncthreads();  // every thread has read the length before it moves
  if (pos < 0 || pos >= max_blocks * BLK) return;  // full (or invalid): nothing written
  const int page = table[s * (int64_t)max_blocks + pos / BLK];
  if (page < 0 || page >= n_pages) return;
  const int slot = pos % BLK;
  for (int e = tid; e < Hkv * D; e += 256) {
    const int g = e / D, dd = e % D;
    const int64_t tile = ((int64_t)page * Hkv + g) * BLK * D;
    const uint16_t kv = k_new[(s * Hkv + g) * D + dd];
    kp[tile + (int64_t)slot * D + dd] = kv;
    vp[tile + (int64_t)slot * D + dd] = v_new[(s * Hkv + g) * D + dd];
    // the page's mean over rows 0 .. slot, summed in row order (as
    // paged_means_kernel does): earlier rows from the pool, the new row from
    // the source (no read-after-write of the pool)
    float sum = 0.f;
#pragma unroll 8
    for (int r = 0; r < slot; ++r) sum += __uint_as_float((uint32_t)kp[tile + (int64_t)r * D + dd] << 16);
    sum += __uint_as_float((uint32_t)kv << 16);
    kbar[((int64_t)page * Hkv + g) * D + dd] = sum / (float)(slot + 1);
  }
  __syncthreads();
  if (tid == 0) lengths[s] = pos + 1;
}

// ============================================================== per-page means
template <int D, int BLK>
__global__ __launch_bounds__(256) void paged_means_kernel(const uint16_t* __restrict__ kp,
                                                          const int32_t* __restrict__ table,
                                                          const int32_t* __restrict__ lengths,
                                                          float* __restrict__ kbar, int S, int Hkv, int max_blocks,
                                                          int n_pages) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w >= (int64_t)S * max_blocks * Hkv) return;
  const int g = (int)(w % Hkv);
  const int64_t sj = w / Hkv;
  const int j = (int)(sj % max_blocks);
  const int64_t s = sj / max_blocks;
  const int L = min(max(lengths[s], 0), max_blocks * BLK);
  if (j * BLK >= L) return;
  const int page = table[s * (int64_t)max_blocks + j];
  if (page < 0 || page >= n_pages) return;
  const int rows = min(BLK, L - j * BLK);
  const uint16_t* tile = kp + ((int64_t)page * Hkv + g) * BLK * D + lane * DPL;
  float acc[DPL] = {};
  for (int r = 0; r < rows; ++r) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] += __uint_as_float((uint32_t)tile[(int64_t)r * D + e] << 16);
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) kbar[((int64_t)page * Hkv + g) * D + lane * DPL + e] = acc[e] / (float)rows;
}

// ============================================================== FP8 cache rows
// One row (D values, D/64 per lane) -> E4M3 codes with scale = amax / 448
// (1 for an all-zero row): codes = round-to-nearest-even of fp32(x / scale),
// by the hardware conversion.  Returns the scale; writes the lane's codes.
template <int D>
__device__ __forceinline__ float quantize_row(const float (&x)[D / 64], uint8_t* out) {
  constexpr int DPL = D / 64;
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = wave_max_f32(amax);
  const float scale = amax > 0.f ? amax / 448.f : 1.f;
  typedef short s2 __attribute__((ext_vector_type(2)));
  const s2 c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((s2){0, 0}, x[0] / scale, DPL == 2 ? x[DPL - 1] / scale : 0.f,
                                                        1.0f, false);
  const uint32_t w = __builtin_bit_cast(uint32_t, c);
  if constexpr (DPL == 2) *reinterpret_cast<uint16_t*>(out) = (uint16_t)(w & 0xffffu);
  else *out = (uint8_t)(w & 0xffu);
  return scale;
}

// the lane's D/64 dequantized values (code * scale) of a row
template <int D>
__device__ __forceinline__ void dequant_row(const uint8_t* codes, float scale, float (&v)[D / 64]) {
  constexpr int DPL = D / 64;
  const int w = DPL == 2 ? (int)*reinterpret_cast<const uint16_t*>(codes) : (int)*codes;
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
#pragma unroll
  for (int e = 0; e < DPL; ++e) v[e] = b[e] * scale;
}

// every slot of every (page, head) tile: one wave per (page, head)
template <int D, int BLK>
__global__ __launch_bounds__(256) void paged_quantize_kernel(const uint16_t* __restrict__ kp,
                                                             const uint16_t* __restrict__ vp, uint8_t* __restrict__ k8,
                                                             uint8_t* __restrict__ v8, float* __restrict__ ksc,
                                                             float* __restrict__ vsc, int64_t n_tiles) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= n_tiles) return;  // whole wave
  for (int r = 0; r < BLK; ++r) {
    const int64_t row = t * BLK + r;
    float x[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) x[e] = __uint_as_float((uint32_t)kp[row * D + lane * DPL + e] << 16);
    float sk = quantize_row<D>(x, k8 + row * D + lane * DPL);
#pragma unroll
    for (int e = 0; e < DPL; ++e) x[e] = __uint_as_float((uint32_t)vp[row * D + lane * DPL + e] << 16);
    float sv = quantize_row<D>(x, v8 + row * D + lane * DPL);
    if (lane == 0) {
      ksc[row] = sk;
      vsc[row] = sv;
    }
  }
}

// append to an FP8 cache: one workgroup per sequence, one wave per KV head
// (4 waves, heads strided); the page mean is recomputed from the dequantized
// rows in row order, as paged_means_fp8_kernel does
template <int D, int BLK>
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(const uint16_t* __restrict__ k_new,
                                                            const uint16_t* __restrict__ v_new,
                                                            const int32_t* __restrict__ table, int32_t* lengths,
                                                            uint8_t* __restrict__ k8, uint8_t* __restrict__ v8,
                                                            float* __restrict__ ksc, float* __restrict__ vsc,
                                                            float* __restrict__ kbar, int Hkv, int max_blocks,
                                                            int n_pages) {
  constexpr int DPL = D / 64;
  const int64_t s = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pos = lengths[s];
  __syncthreads();  // every thread has read the length before it moves
  if (pos < 0 || pos >= max_blocks * BLK) return;
  const int page = table[s * (int64_t)max_blocks + pos / BLK];
  if (page < 0 || page >= n_pages) return;
  const int slot = pos % BLK;
  for (int g = wave; g < Hkv; g += 4) {
    const int64_t tile = ((int64_t)page * Hkv + g) * BLK;  // row index of slot 0
    float x[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) x[e] = __uint_as_float((uint32_t)k_new[(s * Hkv + g) * D + lane * DPL + e] << 16);
    const float sk = quantize_row<D>(x, k8 + (tile + slot) * D + lane * DPL);
#pragma unroll
    for (int e = 0; e < DPL; ++e) x[e] = __uint_as_float((uint32_t)v_new[(s * Hkv + g) * D + lane * DPL + e] << 16);
    const float sv = quantize_row<D>(x, v8 + (tile + slot) * D + lane * DPL);
    if (lane == 0) {
      ksc[tile + slot] = sk;
      vsc[tile + slot] = sv;
    }
    // mean of rows 0 .. slot (the new row's codes are re-read by the lane that wrote them)
    float acc[DPL] = {};
    for (int r = 0; r < slot; ++r) {
      float v[DPL];
      dequant_row<D>(k8 + (tile + r) * D + lane * DPL, ksc[tile + r], v);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += v[e];
    }
    {
      float v[DPL];
      dequant_row<D>(k8 + (tile + slot) * D + lane * DPL, sk, v);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += v[e];
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) kbar[((int64_t)page * Hkv + g) * D + lane * DPL + e] = acc[e] / (float)(slot + 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) lengths[s] = pos + 1;
}

template <int D, int BLK>
__global__ __launch_bounds__(256) void paged_means_fp8_kernel(const uint8_t* __restrict__ k8,
                                                              const float* __restrict__ ksc,
                                                              const int32_t* __restrict__ table,
                                                              const int32_t* __restrict__ lengths,
                                                              float* __restrict__ kbar, int S, int Hkv, int max_blocks,
                                                              int n_pages) {
  constexpr int DPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w >= (int64_t)S * max_blocks * Hkv) return;
  const int g = (int)(w % Hkv);
  const int64_t sj = w / Hkv;
  const int j = (int)(sj % max_blocks);
  const int64_t s = sj / max_blocks;
  const int L = min(max(lengths[s], 0), max_blocks * BLK);
  if (j * BLK >= L) return;
  const int page = table[s * (int64_t)max_blocks + j];
  if (page < 0 || page >= n_pages) return;
  const int rows = min(BLK, L - j * BLK);
  const int64_t tile = ((int64_t)page * Hkv + g) * BLK;
  float acc[DPL] = {};
  for (int r = 0; r < rows; ++r) {
    float v[DPL];
    dequant_row<D>(k8 + (tile + r) * D + lane * DPL, ksc[tile + r], v);
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] += v[e];
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) kbar[((int64_t)page * Hkv + g) * D + lane * DPL + e] = acc[e] / (float)rows;
}

// ============================================================== launch
template <int D, int BLK, bool F8>
static hipError_t launch_paged_d(const PagedArgs& a, TopkParams p, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const dim3 grid((uint32_t)((int64_t)a.S * a.Hkv)), blk(512);
#define DSA_PAGED(GG, RR) hipLaunchKernelGGL((decode_paged_kernel<D, BLK, GG, RR, F8>), grid, blk, 0, stream, a, p)
#define DSA_PAGED_G(RR)                 \
  switch (G) {                          \
    case 1: DSA_PAGED(1, RR); break;    \
    case 2: DSA_PAGED(2, RR); break;    \
    case 4: DSA_PAGED(4, RR); break;    \
    case 8: DSA_PAGED(8, RR); break;    \
    default: return hipErrorInvalidValue; \
  }
  if (a.max_blocks <= 64 * 16) {
    DSA_PAGED_G(16)
  } else {
    DSA_PAGED_G(64)
  }
#undef DSA_PAGED_G
#undef DSA_PAGED
  return hipGetLastError();
}

template <bool F8>
static hipError_t launch_paged_f(const PagedArgs& a, int d, int block, TopkParams p, hipStream_t stream) {
  if (d == 64)
    return block == 64 ? launch_paged_d<64, 64, F8>(a, p, stream) : launch_paged_d<64, 128, F8>(a, p, stream);
  return block == 64 ? launch_paged_d<128, 64, F8>(a, p, stream) : launch_paged_d<128, 128, F8>(a, p, stream);
}

hipError_t launch_paged_decode(const PagedArgs& a, int d, int block, TopkParams p, hipStream_t stream) {
  if ((int64_t)a.S * a.Hkv == 0) return hipSuccess;
  return a.k8 ? launch_paged_f<true>(a, d, block, p, stream) : launch_paged_f<false>(a, d, block, p, stream);
}

hipError_t launch_kv_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* table, int32_t* lengths,
                            uint16_t* kp, uint16_t* vp, float* kbar, int S, int Hkv, int d, int block, int max_blocks,
                            int n_pages, hipStream_t stream) {
  if (S == 0) return hipSuccess;
  const dim3 grid((uint32_t)S), blk(256);
  if (d == 64 && block == 64)
    hipLaunchKernelGGL((kv_append_kernel<64, 64>), grid, blk, 0, stream, k_new, v_new, table, lengths, kp, vp, kbar,
                       Hkv, max_blocks, n_pages);
  else if (d == 64)
    hipLaunchKernelGGL((kv_append_kernel<64, 128>), grid, blk, 0, stream, k_new, v_new, table, lengths, kp, vp, kbar,
                       Hkv, max_blocks, n_pages);
  else if (block == 64)
    hipLaunchKernelGGL((kv_append_kernel<128, 64>), grid, blk, 0, stream, k_new, v_new, table, lengths, kp, vp, kbar,
                       Hkv, max_blocks, n_pages);
  else
    hipLaunchKernelGGL((kv_append_kernel<128, 128>), grid, blk, 0, stream, k_new, v_new, table, lengths, kp, vp, kbar,
                       Hkv, max_blocks, n_pages);
  return hipGetLastError();
}

hipError_t launch_paged_means(const uint16_t* kp, const int32_t* table, const int32_t* lengths, float* kbar, int S,
                              int Hkv, int d, int block, int max_blocks, int n_pages, hipStream_t stream) {
  const int64_t waves = (int64_t)S * max_blocks * Hkv;
  if (waves == 0) return hipSuccess;
  const dim3 grid((uint32_t)((waves + 3) / 4)), blk(256);
  if (d == 64 && block == 64)
    hipLaunchKernelGGL((paged_means_kernel<64, 64>), grid, blk, 0, stream, kp, table, lengths, kbar, S, Hkv,
                       max_blocks, n_pages);
  else if (d == 64)
    hipLaunchKernelGGL((paged_means_kernel<64, 128>), grid, blk, 0, stream, kp, table, lengths, kbar, S, Hkv,
                       max_blocks, n_pages);
  else if (block == 64)
    hipLaunchKernelGGL((paged_means_kernel<128, 64>), grid, blk, 0, stream, kp, table, lengths, kbar, S, Hkv,
                       max_blocks, n_pages);
  else
    hipLaunchKernelGGL((paged_means_kernel<128, 128>), grid, blk, 0, stream, kp, table, lengths, kbar, S, Hkv,
                       max_blocks, n_pages);
  return hipGetLastError();
}

#define DSA_DB(F, ...)                                                  \
  if (d == 64 && block == 64) hipLaunchKernelGGL((F<64, 64>), __VA_ARGS__); \
  else if (d == 64) hipLaunchKernelGGL((F<64, 128>), __VA_ARGS__);          \
  else if (block == 64) hipLaunchKernelGGL((F<128, 64>), __VA_ARGS__);      \
  else hipLaunchKernelGGL((F<128, 128>), __VA_ARGS__)

hipError_t launch_paged_quantize(const uint16_t* kp, const uint16_t* vp, uint8_t* k8, uint8_t* v8, float* ksc,
                                 float* vsc, int n_pages, int Hkv, int d, int block, hipStream_t stream) {
  const int64_t tiles = (int64_t)n_pages * Hkv;
  if (tiles == 0) return hipSuccess;
  const dim3 grid((uint32_t)((tiles + 3) / 4)), blk(256);
  DSA_DB(paged_quantize_kernel, grid, blk, 0, stream, kp, vp, k8, v8, ksc, vsc, tiles);
  return hipGetLastError();
}

hipError_t launch_kv_append_fp8(const uint16_t* k_new, const uint16_t* v_new, const int32_t* table, int32_t* lengths,
                                uint8_t* k8, uint8_t* v8, float* ksc, float* vsc, float* kbar, int S, int Hkv, int d,
                                int block, int max_blocks, int n_pages, hipStream_t stream) {
  if (S == 0) return hipSuccess;
  const dim3 grid((uint32_t)S), blk(256);
  DSA_DB(kv_append_fp8_kernel, grid, blk, 0, stream, k_new, v_new, table, lengths, k8, v8, ksc, vsc, kbar, Hkv,
         max_blocks, n_pages);
  return hipGetLastError();
}

hipError_t launch_paged_means_fp8(const uint8_t* k8, const float* ksc, const int32_t* table, const int32_t* lengths,
                                  float* kbar, int S, int Hkv, int d, int block, int max_blocks, int n_pages,
                                  hipStream_t stream) {
  const int64_t waves = (int64_t)S * max_blocks * Hkv;
  if (waves == 0) return hipSuccess;
  const dim3 grid((uint32_t)((waves + 3) / 4)), blk(256);
  DSA_DB(paged_means_fp8_kernel, grid, blk, 0, stream, k8, ksc, table, lengths, kbar, S, Hkv, max_blocks, n_pages);
  return hipGetLastError();
}
#undef DSA_DB

}  // namespace dsa
