// Sparse attention backward over the selected key blocks: dQ, dK, dV with the
// selection held fixed (bf16 MFMA, fp32 accumulation).
//
// Method: "稀疏注意力 vs Flash Attention v2" (pnsm.cn/news/1249548.html),
// section 1, defines the forward (softmax of the scaled logits over the kept
// keys, times V) and notes that FlashAttention-2 recomputes rather than
// stores the score matrix; the backward is the chain rule through that
// forward, recomputing P from the saved log-sum-exp:
//   P = exp(s q k^T - lse),  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dQ = s dS K,  dK = s dS^T Q,  dV = P^T dO   (s = 1/sqrt(d), GQA: dK/dV summed
//   over the group's query heads).
//
// Launches (all on the caller's stream):
//   1. bwd_prep_kernel: D per query row (fp32), d/8 lanes per row with DPP sums;
//   2. bwd_invert_kernel: for every KV block j the ascending list of query
//      blocks whose selection kept j (one wave per j, membership by binary
//      search in the sorted index rows, compaction by ballot);
//   3. bwd_dq_kernel: one workgroup per (batch, KV head, HG query heads, query
//      block), each wave 32 query rows, walking the kept tiles like the
//      forward: S^T = K Q^T and dP^T = V dO^T (K, V rows from LDS as A
//      operands, Q^T and dO^T in registers as B), dS^T in registers, then
//      dQ^T += K^T dS^T with K^T from transposed LDS reads.  K is used at both
//      ends of a tile, so it is double-buffered; V is single-buffered.  Two
//      barriers per tile;
//   4. bwd_dkdv_kernel: one workgroup per (batch, KV head, KV block), each
//      wave 32 keys (64-key blocks: two waves per key group, each taking half
//      of every query tile, added at the end); the waves' K and V operands
//      sit in registers, and for every (query block of the inverted list) x
//      (query head of the group) the Q and dO tiles stream through
//      a ring of LDS stages: S = Q K^T, dP = dO V^T (Q, dO rows as A operands,
//      K, V as B), P and dS in registers (already in B-operand order), then
//      dV^T += dO^T P and dK^T += Q^T dS with dO^T, Q^T from transposed LDS
//      reads.
// Tiles in LDS are read row-wise, and Q, dO and K also transposed; all use
// qswz, which keeps both kinds of read free of bank conflicts.
#include "attn_common.hpp"

namespace dsa {

// ============================================================== tile loads
// A ROWS x D bf16 tile (rows row0 .. row0 + ROWS - 1 of a [*, D] matrix,
// rows clamped to n_rows - 1) into LDS with the qswz layout, by WAVES waves.
template <int D, int ROWS, int WAVES>
__device__ __forceinline__ void load_tile(const uint16_t* g, int row0, int n_rows, uint32_t lds_base, int wave,
                                          int lane) {
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int RPI = 1024 / (2 * D);    // rows per 1 KiB wave load
  constexpr int LOADS = ROWS * D * 2 / 1024;
  static_assert(LOADS % WAVES == 0, "tile loads must split evenly over waves");
#pragma unroll
  for (int n = 0; n < LOADS / WAVES; ++n) {
    const int inst = wave + n * WAVES;
    const int r = inst * RPI + lane / CH;
    const int c = (lane % CH) ^ qswz<D>(r);
    const int row = min(row0 + r, n_rows - 1);
    dma16(g, (uint32_t)(row * D + c * 8) * 2u, __builtin_amdgcn_readfirstlane(lds_base + inst * 1024));
  }
}

// 8 bf16 of the transposed operand: rows t0 + {0..3} and t0 + 8 + {0..3} of
// a qswz tile at column block `d` (lane layout of ds_read_b64_tr_b16: within
// 16 lanes, out lane i slot j receives element i % 4 of source lane 4j + i/4;
// source lane s reads row base + s / 4, columns dbase + 4 (s % 4) .. + 3).
template <int D>
__device__ __forceinline__ u32x4 read_tr(const LDS_AS uint16_t* tile, int row_base, int d) {
  u32x4 f;
  const int cbase = d >> 3, sub = (d & 7) * 2;  // 16-byte chunk and byte offset (0 or 8)
#pragma unroll
  for (int sg = 0; sg < 2; ++sg) {
    const int row = row_base + 8 * sg;
    const int c = cbase ^ qswz<D>(row);
    const LDS_AS char* addr = reinterpret_cast<const LDS_AS char*>(tile + row * D + c * 8) + sub;
    const i16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)addr);
    const u32x2 w = __builtin_bit_cast(u32x2, v4);
    f[2 * sg] = w[0];
    f[2 * sg + 1] = w[1];
  }
  return f;
}

// row-major operand fragment: row r, k-step ks (dims 16 ks + 8 half .. + 7)
template <int D>
__device__ __forceinline__ u32x4 read_row(const LDS_AS uint16_t* tile, int r, int ks, int half) {
  const int c = (2 * ks + half) ^ qswz<D>(r);
  return *reinterpret_cast<const LDS_AS u32x4*>(tile + r * D + c * 8);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const bf16x2_t pk = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, pk);
}

// ============================================================== 1. row statistics
// rowstat[bh][i][0][r] = lse * log2(e), rowstat[bh][i][1][r] = rowsum(dO * O)
// for row i BLK + r of head bh; rows past N (the ragged last block) get zeros.
// d/8 lanes per row (cross-lane sums); each thread takes four rows, issuing
// all their loads before any sum.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ lse, float* __restrict__ rowstat,
                                                       int64_t n_pad_rows, int N, int BLK, int nB) {
  constexpr int TPR = D / 8, RPP = 256 / TPR;  // lanes per row, rows per pass
  constexpr int PASSES = 4;                     // rows per thread, all loads issued first
  const int c = threadIdx.x % TPR;
  const int64_t npad = (int64_t)nB * BLK;
  u32x4 x[PASSES], y[PASSES];
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    const int64_t prow = ((int64_t)blockIdx.x * PASSES + k) * RPP + threadIdx.x / TPR;  // bh * nB BLK + n
    const int64_t bh = prow / npad;
    const int n = (int)(prow % npad);
    x[k] = y[k] = (u32x4){0u, 0u, 0u, 0u};
    if (prow < n_pad_rows && n < N) {
      const int64_t row = bh * N + n;
      x[k] = *reinterpret_cast<const u32x4*>(o + row * D + 8 * c);
      y[k] = *reinterpret_cast<const u32x4*>(dout + row * D + 8 * c);
    }
  }
#pragma unroll
  for (int k = 0; k < PASSES; ++k) {
    const int64_t prow = ((int64_t)blockIdx.x * PASSES + k) * RPP + threadIdx.x / TPR;
    const int64_t bh = prow / npad;
    const int n = (int)(prow % npad);
    const bool real = prow < n_pad_rows && n < N;
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bf16_lo(x[k][e]) * bf16_lo(y[k][e]) + bf16_hi(x[k][e]) * bf16_hi(y[k][e]);
#pragma unroll
    for (int off = 1; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
    if (prow < n_pad_rows && c == 0) {
      float* st = rowstat + (bh * nB + n / BLK) * 2 * BLK + n % BLK;
      st[0] = real ? lse[bh * N + n] * 1.4426950408889634f : 0.f;
      st[BLK] = acc;
    }
  }
}

// ============================================================== 2. inverted selection
// One wave per (unit, KV block j): query blocks i >= j in chunks of 64 lanes;
// lane i keeps i if j is in the sorted row idx[i][0 .. cnt_i).
__global__ __launch_bounds__(256) void bwd_invert_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
                                                         int32_t* __restrict__ inv_cnt, int32_t* __restrict__ inv_idx,
                                                         int64_t n_waves, int nB, int kmax) {
  const int64_t w = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w >= n_waves) return;
  const int lane = threadIdx.x & 63;
  const int64_t unit = w / nB;
  const int j = (int)(w % nB);
  int32_t* out = inv_idx + w * nB;
  int total = 0;
  for (int i0 = j; i0 < nB; i0 += 64) {
    const int i = i0 + lane;
    bool hit = false;
    if (i < nB) {
      const int32_t* row = idx + (unit * nB + i) * (int64_t)kmax;
      // count and block ids clamped into range, as where the forward and
      // the dQ kernel read them (clamping keeps an ascending row ascending)
      const int n = min(max(cnt[unit * nB + i], 0), kmax);
      auto at = [&](int e) { return min(max(row[e], 0), nB - 1); };
      int lo = 0, hi = n;  // ascending block ids
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (at(mid) < j) lo = mid + 1;
        else hi = mid;
      }
      hit = lo < n && at(lo) == j;
    }
    const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
    if (hit) out[total + below] = i;
    total += __builtin_popcountll(m);
  }
  if (lane == 0) inv_cnt[w] = total;
}

// ============================================================== 3. dQ
template <int D, int BLK, int HG>
struct BwdQCfg {
  static constexpr int SLABS = BLK / 32;
  static constexpr int WAVES = HG * SLABS;
  static constexpr int THREADS = WAVES * 64;
};

template <int D, int BLK, int HG>
__global__ __launch_bounds__((BwdQCfg<D, BLK, HG>::THREADS)) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(BwdArgs a) {
  using C = BwdQCfg<D, BLK, HG>;
  constexpr int NKS = D / 16, NST = BLK / 32;
  __shared__ __align__(1024) uint16_t Ks[2][BLK * D];
  __shared__ __align__(1024) uint16_t Vs[BLK * D];

  const int G = a.Hq / a.Hkv;
  const int hchunks = G / HG;
  const uint32_t L = xcd_logical_id(blockIdx.x, gridDim.x);
  const int i = a.nB - 1 - (int)(L % (uint32_t)a.nB);
  const uint32_t u = L / (uint32_t)a.nB;
  const int hc = (int)(u % (uint32_t)hchunks);
  const int64_t bg = u / (uint32_t)hchunks;
  const int64_t b = bg / a.Hkv;
  const int g = (int)(bg % a.Hkv);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = wave / C::SLABS, slab = wave % C::SLABS;
  const int h = g * G + hc * HG + hl;
  const int half = lane >> 5;
  const int row_in_blk = slab * 32 + (lane & 31);
  const int row = i * BLK + row_in_blk;
  const int N = a.N;
  const int64_t qrow = (b * a.Hq + h) * (int64_t)N + min(row, N - 1);

  const uint16_t* kgp = a.k + bg * (int64_t)N * D;
  const uint16_t* vgp = a.v + bg * (int64_t)N * D;
  const CONST_AS int32_t* irow = (const CONST_AS int32_t*)(a.idx + (bg * a.nB + i) * (int64_t)a.kmax);
  // counts and block ids clamped into range (as in the forward)
  const int n_sel = min(max(((const CONST_AS int32_t*)a.cnt)[bg * a.nB + i], 0), a.kmax);
  auto blk_at = [&](int t) { return min(max(irow[t], 0), a.nB - 1); };
  const uint32_t kbase[2] = {(uint32_t)(uintptr_t)(LDS_AS uint16_t*)Ks[0], (uint32_t)(uintptr_t)(LDS_AS uint16_t*)Ks[1]};
  const uint32_t vbase = (uint32_t)(uintptr_t)(LDS_AS uint16_t*)Vs;

  if (n_sel > 0) {
    load_tile<D, BLK, C::WAVES>(kgp, blk_at(0) * BLK, N, kbase[0], wave, lane);
    load_tile<D, BLK, C::WAVES>(vgp, blk_at(0) * BLK, N, vbase, wave, lane);
  }
  // B operands: lane's row, dims 16 ks + 8 half .. + 7
  u32x4 qf[NKS], df[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = *reinterpret_cast<const u32x4*>(a.q + qrow * D + ks * 16 + 8 * half);
    df[ks] = *reinterpret_cast<const u32x4*>(a.dout + qrow * D + ks * 16 + 8 * half);
  }
  const float* stat = a.rowstat + ((b * a.Hq + h) * a.nB + i) * 2 * BLK + row_in_blk;
  const float lse2 = stat[0];  // log2 units
  const float drow = stat[BLK];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(qf[ks]), "v"(df[ks]));
  asm volatile("" ::"v"(lse2), "v"(drow));

  f32x16 dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dq[dt] = (f32x16){};
  const float c2 = a.scale_log2;

  for (int t = 0; t < n_sel; ++t) {
    const int j = blk_at(t);
    const bool more = t + 1 < n_sel;
    const int jn = more ? blk_at(t + 1) : 0;
    const LDS_AS uint16_t* ks_l = (const LDS_AS uint16_t*)Ks[t & 1];
    // ---- K(t), V(t) resident; every wave is done with tile t - 1
    wait_vm<0>();
    __syncthreads();
    if (more) load_tile<D, BLK, C::WAVES>(kgp, jn * BLK, N, kbase[(t + 1) & 1], wave, lane);
    // ---- S^T = K Q^T, dP^T = V dO^T
    f32x16 s[NST], dp[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) s[st] = dp[st] = (f32x16){};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int kr = st * 32 + (lane & 31);
        s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(read_row<D>(ks_l, kr, ks, half)), as_bf16x8(qf[ks]),
                                                        s[st], 0, 0, 0);
        dp[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            as_bf16x8(read_row<D>((const LDS_AS uint16_t*)Vs, kr, ks, half)), as_bf16x8(df[ks]), dp[st], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done reading V(t)
    if (more) load_tile<D, BLK, C::WAVES>(vgp, jn * BLK, N, vbase, wave, lane);
    // ---- dS^T = P^T (dP^T - D), P^T = exp2(s c2 - lse2), causal mask on the diagonal
    const int k_hi = (j == i) ? row_in_blk : BLK;  // kept keys: key_in_blk <= k_hi
    u32x4 dsf[BLK / 16];
#pragma unroll
    for (int kk = 0; kk < BLK / 16; ++kk) {
      const int st = kk >> 1, rb = 8 * (kk & 1);
      float v8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = rb + e;
        const int key_in_blk = st * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][r], c2, -lse2));
        v8[e] = (key_in_blk <= k_hi ? p : 0.f) * (dp[st][r] - drow);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) dsf[kk][e] = pack2(v8[2 * e], v8[2 * e + 1]);
    }
    // ---- dQ^T += K^T dS^T (K^T by transposed reads)
    {
      const int grp = (lane >> 4) & 1, si = lane & 15;
#pragma unroll
      for (int kk = 0; kk < BLK / 16; ++kk) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int d = dt * 32 + 16 * grp + 4 * (si & 3);
          const u32x4 kf = read_tr<D>(ks_l, 16 * kk + 4 * half + (si >> 2), d);
          dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(dsf[kk]), dq[dt], 0, 0, 0);
        }
      }
    }
  }
  wait_vm<0>();

  // ---- dQ = s dS K (bf16)
  if (row < N) {
    uint16_t* orow = a.dq + ((b * a.Hq + h) * (int64_t)N + row) * D;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 w;
        w[0] = pack2(dq[dt][4 * q4 + 0] * sc, dq[dt][4 * q4 + 1] * sc);
        w[1] = pack2(dq[dt][4 * q4 + 2] * sc, dq[dt][4 * q4 + 3] * sc);
        *reinterpret_cast<u32x2*>(orow + dt * 32 + 8 * q4 + 4 * half) = w;
      }
    }
  }
}

// ============================================================== 4. dK, dV
// Waves: KG = BLK / 32 key groups (32 keys each) x QS query splits (2 for
// 64-row tiles, 1 for 128); a wave accumulates dK^T, dV^T of its keys over
// its share of every query tile, and the splits are added at the end.  A
// work item (query tile of one head) is a Q tile, a dO tile and its row
// statistics; NBUF of them are in flight in LDS.
template <int D, int BLK>
struct BwdKVCfg {
  static constexpr int KG = BLK / 32;
  static constexpr int QS = BLK == 64 ? 2 : 1;
  static constexpr int WAVES = KG * QS;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int QB_PER_WAVE = (BLK / 32) / QS;  // 32-query sub-blocks per wave per tile
  static constexpr int TILE = BLK * D;                  // bf16 elements
  static constexpr int STAGE_BYTES = 2 * TILE * 2 + 2 * BLK * 4;
  // as many stages (up to 4) as 136 KiB of LDS holds: one workgroup per CU
  // either way, and a deeper ring keeps more item loads in flight
  static constexpr int NBUF = 4 * STAGE_BYTES <= 136 * 1024 ? 4 : 3 * STAGE_BYTES <= 136 * 1024 ? 3 : 2;
  static constexpr int STAT_BYTES_PER_WAVE = 2 * BLK * 4 / WAVES;  // statistics DMA: one instruction per wave
  static constexpr int LOADS_PER_ITEM = 2 * (TILE * 2 / 1024) / WAVES + 1;  // DMA instructions per wave
  // dV/dK steps (one dO^T and one Q^T fragment each) read ahead of their
  // MFMAs; 128-key blocks already use every VGPR, so they look less far
  static constexpr int DVK_LOOK = BLK == 64 ? 4 : 2;
  static_assert(STAT_BYTES_PER_WAVE % 16 == 0 && STAT_BYTES_PER_WAVE <= 1024, "statistics split");
};

template <int D, int BLK>
__global__ __launch_bounds__((BwdKVCfg<D, BLK>::THREADS)) void bwd_dkdv_kernel(BwdArgs a) {
  using C = BwdKVCfg<D, BLK>;
  constexpr int NKS = D / 16, NBUF = C::NBUF;
  // stage s: Q tile tiles[s][0], dO tile tiles[s][1], statistics stats[s]
  __shared__ __align__(1024) uint16_t tiles[NBUF][2][C::TILE];
  __shared__ __align__(16) float stats[NBUF][2 * BLK];  // lse log2(e), then D

  // key-block-major order: the long lists of the first blocks (the sink is
  // kept by every query block) start first; a unit's blocks share an XCD
  const int64_t n_units = (int64_t)a.B * a.Hkv;
  const int j = (int)(blockIdx.x / n_units);
  const int64_t bg = blockIdx.x % n_units;  // b * Hkv + g
  const int64_t wl = bg * a.nB + j;         // this block's inverted list
  const int64_t b = bg / a.Hkv;
  const int g = (int)(bg % a.Hkv);
  const int G = a.Hq / a.Hkv;
  const int N = a.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave % C::KG, qs = wave / C::KG;
  const int half = lane >> 5;
  const int key_in_blk = kg * 32 + (lane & 31);
  const int key = j * BLK + key_in_blk;
  const int64_t krow = bg * (int64_t)N + min(key, N - 1);

  // B operands of this wave's keys (column = key, k-slots = dims 16 ks + 8 half ..)
  u32x4 kf[NKS], vf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kf[ks] = *reinterpret_cast<const u32x4*>(a.k + krow * D + ks * 16 + 8 * half);
    vf[ks] = *reinterpret_cast<const u32x4*>(a.v + krow * D + ks * 16 + 8 * half);
  }
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(kf[ks]), "v"(vf[ks]));

  const int n_list = a.inv_cnt[wl];
  const CONST_AS int32_t* list = (const CONST_AS int32_t*)(a.inv_idx + wl * a.nB);
  const int n_work = n_list * G;
  const float c2 = a.scale_log2;

  // work item w: query block list[w / G], query head g G + w % G, stage w % NBUF.
  // Every wave issues exactly LOADS_PER_ITEM DMA instructions per item.
  auto issue = [&](int w) {
    const int i = list[w / G];
    const int h = g * G + w % G;
    const int64_t bh = b * a.Hq + h;
    const int sg = w % NBUF;
    const int64_t hrow0 = bh * (int64_t)N;
    load_tile<D, BLK, C::WAVES>(a.q + hrow0 * D, i * BLK, N, (uint32_t)(uintptr_t)(LDS_AS uint16_t*)tiles[sg][0],
                                wave, lane);
    load_tile<D, BLK, C::WAVES>(a.dout + hrow0 * D, i * BLK, N, (uint32_t)(uintptr_t)(LDS_AS uint16_t*)tiles[sg][1],
                                wave, lane);
    const float* st = a.rowstat + (bh * a.nB + i) * 2 * BLK;
    const uint32_t off = (uint32_t)(wave * C::STAT_BYTES_PER_WAVE);
    if (lane < C::STAT_BYTES_PER_WAVE / 16)
      dma16(st, off + 16u * (uint32_t)lane,
            __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS float*)stats[sg] + off));
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dk[dt] = dv[dt] = (f32x16){};

#pragma unroll
  for (int w = 0; w < NBUF - 1; ++w)
    if (w < n_work) issue(w);
  for (int w = 0; w < n_work; ++w) {
    const int sg = w % NBUF;
    const int i = list[w / G];
    // item w resident: the items issued after it may still be in flight
    if (w + NBUF - 2 < n_work) wait_vm<(NBUF - 2) * C::LOADS_PER_ITEM>();
    else wait_vm<0>();
    __syncthreads();  // every wave is done with item w - 1, whose stage is refilled next
    if (w + NBUF - 1 < n_work) issue(w + NBUF - 1);
    const LDS_AS uint16_t* qs_l = (const LDS_AS uint16_t*)tiles[sg][0];
    const LDS_AS uint16_t* os_l = (const LDS_AS uint16_t*)tiles[sg][1];
    const LDS_AS float* st_l = (const LDS_AS float*)stats[sg];
    // kept: query >= key on the diagonal block, query < N (branch-free)
    const int q_lo = (i == j) ? key_in_blk : 0;
    const int q_hi = N - i * BLK;
    // kept rolled: unrolled, the sub-blocks' statistics and addresses are
    // hoisted together and leave no registers to read Q and dO rows ahead
#pragma nounroll
    for (int qq = 0; qq < C::QB_PER_WAVE; ++qq) {
      const int qb = qs * C::QB_PER_WAVE + qq;
      const int qr = qb * 32 + (lane & 31);
      // statistics of this lane's 16 query rows: qb 32 + 8 t + 4 half + {0..3}
      f32x4 lse4[4], d4[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lse4[t] = *reinterpret_cast<const LDS_AS f32x4*>(st_l + qb * 32 + 8 * t + 4 * half);
        d4[t] = *reinterpret_cast<const LDS_AS f32x4*>(st_l + BLK + qb * 32 + 8 * t + 4 * half);
      }
      // S = Q K^T, dP = dO V^T (M = queries, N = keys); Q, dO row reads one
      // k-step ahead of their MFMAs
      f32x16 sacc = (f32x16){}, dpacc = (f32x16){};
      u32x4 qa = read_row<D>(qs_l, qr, 0, half), oa = read_row<D>(os_l, qr, 0, half);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 qn = qa, on = oa;
        if (ks + 1 < NKS) {
          qn = read_row<D>(qs_l, qr, ks + 1, half);
          on = read_row<D>(os_l, qr, ks + 1, half);
        }
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa), as_bf16x8(kf[ks]), sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(oa), as_bf16x8(vf[ks]), dpacc, 0, 0, 0);
        qa = qn;
        oa = on;
      }
      // dV/dK step st = (kk, dt) multiplies transposed dO and Q fragments;
      // they are read DVK_LOOK steps ahead, the first ones before P and dS
      // are formed so that their latency hides behind that arithmetic (at
      // one wave per SIMD nothing else hides it)
      constexpr int NST = 2 * (D / 32), LOOK = C::DVK_LOOK < NST ? C::DVK_LOOK : NST;
      const int grp = (lane >> 4) & 1, si = lane & 15;
      u32x4 fo[NST], fq[NST];
      auto fetch = [&](int st) {
        const int d = (st % (D / 32)) * 32 + 16 * grp + 4 * (si & 3);
        const int rb = qb * 32 + 16 * (st / (D / 32)) + 4 * half + (si >> 2);
        fo[st] = read_tr<D>(os_l, rb, d);
        fq[st] = read_tr<D>(qs_l, rb, d);
      };
      // LDS reads and MFMAs stay on their side of these fences; VALU, SALU
      // and exp may cross
      __builtin_amdgcn_sched_barrier(0x0406);
#pragma unroll
      for (int st = 0; st < LOOK; ++st) fetch(st);
      __builtin_amdgcn_sched_barrier(0x0406);
      // element r: query qb 32 + 8 (r / 4) + 4 half + r % 4, this lane's key.
      // P and dS packed to bf16 in B-operand order (k-chunk kk: elements 8 kk .. 8 kk + 7)
      u32x4 pf[2], sf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float pv[8], dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * kk + e;
          const int q_in_blk = qb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c2, -lse4[r >> 2][r & 3]));
          const bool keep = (q_in_blk >= q_lo) & (q_in_blk < q_hi);
          pv[e] = keep ? p : 0.f;
          dsv[e] = pv[e] * (dpacc[r] - d4[r >> 2][r & 3]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pf[kk][e] = pack2(pv[2 * e], pv[2 * e + 1]);
          sf[kk][e] = pack2(dsv[2 * e], dsv[2 * e + 1]);
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS (M = d, N = keys, K = these 32 queries)
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        if (st + LOOK < NST) fetch(st + LOOK);
        const int kk = st / (D / 32), dt = st % (D / 32);
        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fo[st]), as_bf16x8(pf[kk]), dv[dt], 0, 0, 0);
        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fq[st]), as_bf16x8(sf[kk]), dk[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0x0406);
      }
    }
  }
  wait_vm<0>();

  // ---- add the query splits through LDS (the tile buffers are free now)
  if constexpr (C::QS > 1) {
    static_assert(C::QS == 2, "two query splits");
    static_assert(C::KG * 2 * (D / 32) * 16 * 64 * 4 <= sizeof(tiles), "split merge fits the tile buffers");
    float* red = reinterpret_cast<float*>(&tiles[0][0][0]);  // [kg][dk/dv][dt][r][lane]
    __syncthreads();
    if (qs == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          red[(((kg * 2 + 0) * (D / 32) + dt) * 16 + r) * 64 + lane] = dk[dt][r];
          red[(((kg * 2 + 1) * (D / 32) + dt) * 16 + r) * 64 + lane] = dv[dt][r];
        }
    }
    __syncthreads();
    if (qs == 1) return;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[dt][r] += red[(((kg * 2 + 0) * (D / 32) + dt) * 16 + r) * 64 + lane];
        dv[dt][r] += red[(((kg * 2 + 1) * (D / 32) + dt) * 16 + r) * 64 + lane];
      }
  }

  // ---- dK = s dS^T Q, dV = P^T dO (bf16); a block no row kept gets zeros
  if (key < N) {
    uint16_t* kout = a.dk + (bg * (int64_t)N + key) * D;
    uint16_t* vout = a.dv + (bg * (int64_t)N + key) * D;
    const float sc = a.scale;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2 wk, wv;
        wk[0] = pack2(dk[dt][4 * q4 + 0] * sc, dk[dt][4 * q4 + 1] * sc);
        wk[1] = pack2(dk[dt][4 * q4 + 2] * sc, dk[dt][4 * q4 + 3] * sc);
        wv[0] = pack2(dv[dt][4 * q4 + 0], dv[dt][4 * q4 + 1]);
        wv[1] = pack2(dv[dt][4 * q4 + 2], dv[dt][4 * q4 + 3]);
        *reinterpret_cast<u32x2*>(kout + dt * 32 + 8 * q4 + 4 * half) = wk;
        *reinterpret_cast<u32x2*>(vout + dt * 32 + 8 * q4 + 4 * half) = wv;
      }
    }
  }
}

// ============================================================== launch
hipError_t launch_bwd_prep(const uint16_t* o, const uint16_t* dout, const float* lse, float* rowstat, int64_t n_heads,
                           int N, int d, int block, int nB, hipStream_t stream) {
  const int64_t n_pad_rows = n_heads * nB * (int64_t)block;
  if (n_pad_rows == 0) return hipSuccess;
  const int rows_per_wg = 4 * (256 / (d / 8));  // bwd_prep_kernel: 4 passes of 256 / (d / 8) rows
  const dim3 grid((uint32_t)((n_pad_rows + rows_per_wg - 1) / rows_per_wg)), blk(256);
  if (d == 64)
    hipLaunchKernelGGL(bwd_prep_kernel<64>, grid, blk, 0, stream, o, dout, lse, rowstat, n_pad_rows, N, block, nB);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<128>, grid, blk, 0, stream, o, dout, lse, rowstat, n_pad_rows, N, block, nB);
  return hipGetLastError();
}

hipError_t launch_bwd_invert(const int32_t* idx, const int32_t* cnt, int32_t* inv_cnt, int32_t* inv_idx,
                             int64_t n_units, int nB, int kmax, hipStream_t stream) {
  const int64_t n_waves = n_units * nB;
  if (n_waves == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_invert_kernel, dim3((uint32_t)((n_waves + 3) / 4)), dim3(256), 0, stream, idx, cnt, inv_cnt,
                     inv_idx, n_waves, nB, kmax);
  return hipGetLastError();
}

template <int D, int BLK, int HG>
static hipError_t launch_dq_cfg(const BwdArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const int64_t n_wg = (int64_t)a.B * a.Hkv * (G / HG) * a.nB;
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dq_kernel<D, BLK, HG>), dim3((uint32_t)n_wg), dim3(BwdQCfg<D, BLK, HG>::THREADS), 0, stream,
                     a);
  return hipGetLastError();
}

template <int D, int BLK>
static hipError_t launch_bwd_d_blk(const BwdArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  hipError_t e;
  if constexpr (BLK == 64) {
    if (G % 2 == 0) e = launch_dq_cfg<D, BLK, 2>(a, stream);
    else e = launch_dq_cfg<D, BLK, 1>(a, stream);
  } else {
    e = launch_dq_cfg<D, BLK, 1>(a, stream);
  }
  if (e != hipSuccess) return e;
  const int64_t n_wg = (int64_t)a.B * a.Hkv * a.nB;
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, BLK>), dim3((uint32_t)n_wg), dim3(BwdKVCfg<D, BLK>::THREADS), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_bwd(const BwdArgs& a, int d, int block, hipStream_t stream) {
  if (d == 64) return block == 64 ? launch_bwd_d_blk<64, 64>(a, stream) : launch_bwd_d_blk<64, 128>(a, stream);
  return block == 64 ? launch_bwd_d_blk<128, 64>(a, stream) : launch_bwd_d_blk<128, 128>(a, stream);
}

}  // namespace dsa
