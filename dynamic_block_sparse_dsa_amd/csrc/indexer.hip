// Token-level lightning indexer and token-gather attention (gfx950).
//
// Method: "低成本高性能大模型实现路径：从架构创新到工程优化"
// (yunthe.com/news/806485.html), section 2.1 "轻量化索引器设计": an indexer of
// ReLU feature heads (16 index heads) decides, per query token, which 64
// key/value tokens matter; section 2.2 keeps the indexer's intermediates in
// low precision.  Here the score of earlier token s for query token t is
//   I[t, s] = sum_h w[t, h] * ReLU(qi[t, h] . ki[s])
// (bf16 MFMA, fp32 accumulation), each query token keeps its top-k tokens
// (the block path's one-wave top-k, rows = tokens, sink and self forced), and
// every attention head attends over its token's kept key/value rows.
//
// index_scores_kernel: one workgroup per 16 query tokens, each wave 4 tokens
//   = 2 tiles of 32 (token, index head) pairs.  Per 64-key tile (global ->
//   LDS DMA, double-buffered, kswz rows): S = Qi . K_tile^T on
//   v_mfma_f32_32x32x16_bf16 (the wave's index query rows as A in registers,
//   key rows from LDS as B), so a lane's output holds one key and 8 heads of
//   each of two tokens; ReLU times the head weight is summed over those in
//   the lane, the other 8 heads come from lane l ^ 32, and each lane stores
//   one score (32 consecutive keys of a token per half-wave), causal part
//   only.  Token tiles run latest first (they have the most key tiles).
// token_attn_kernel: one wave per (batch, token, KV head), KV-head-major over
//   XCD-contiguous workgroups (one KV head's rows per XCD L2).  The kept
//   positions arrive 64 at a time (one coalesced load, spread by lane
//   shuffles); each 32-token chunk gathers its K rows in MFMA A-operand layout
//   (16 rows x 64 bytes per wave load) and its V rows as 16-byte pieces of
//   whole rows, two chunks in flight, and runs the decode path's chunk step:
//   Q K^T on v_mfma_f32_16x16x32_bf16 (kept keys x the group's query heads),
//   online softmax in fp32, P V in fp32 VALU.
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
template <int DI>
__global__ __launch_bounds__(256) void index_scores_kernel(const uint16_t* __restrict__ qi,
                                                           const uint16_t* __restrict__ ki,
                                                           const float* __restrict__ wi, float* __restrict__ scores,
                                                           int N, int tiles_per_b) {
  constexpr int HI = 16, NKS = DI / 16, KT = 64, TPW = 4, TPB = 4 * TPW;
  __shared__ __align__(1024) uint16_t kt_lds[2][KT * DI];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, i16 = lane & 15;
  const int64_t b = blockIdx.x / tiles_per_b;
  const int tile = tiles_per_b - 1 - (int)(blockIdx.x % tiles_per_b);
  const int t0 = tile * TPB;
  const int n_kt = (min(t0 + TPB, N) - 1) / KT + 1;

  // A operands: row (lane % 32) of pair tile ct is the (token, index head)
  // pair (t0 + 4 wave + 2 ct + (lane % 32) / 16, lane % 16)
  u32x4 qf[2][NKS];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int tk = t0 + TPW * wave + 2 * ct + ((lane & 31) >> 4);
    const uint16_t* qrow = qi + ((b * N + min(tk, N - 1)) * HI + i16) * DI;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ct][ks] = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + 8 * half);
  }
  // Output register r of lane l holds key l % 32 and pair row
  // 8 (r / 4) + 4 half + r % 4: registers 0..7 are token 2 ct (heads
  // 4 half + r % 4 and 8 + 4 half + r % 4), 8..15 token 2 ct + 1, same heads.
  // wr: the head weight of each register; the lane stores token 2 ct + half.
  float wr[2][16];
  int tok[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tr = t0 + TPW * wave + 2 * ct + (r >> 3);
      const int hd = 8 * ((r >> 2) & 1) + 4 * half + (r & 3);
      wr[ct][r] = wi[(b * N + min(tr, N - 1)) * HI + hd];
    }
    tok[ct] = t0 + TPW * wave + 2 * ct + half;
  }
  const uint16_t* kb = ki + b * (int64_t)N * DI;
  const uint32_t base[2] = {(uint32_t)(uintptr_t)(LDS_AS uint16_t*)kt_lds[0],
                            (uint32_t)(uintptr_t)(LDS_AS uint16_t*)kt_lds[1]};
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(qf[ct][ks]));
  load_key_tile<DI>(kb, 0, N, base[0], wave, lane);

  for (int kt = 0; kt < n_kt; ++kt) {
    wait_vm<0>();
    __syncthreads();  // tile kt resident; every wave is done with tile kt - 1
    if (kt + 1 < n_kt) load_key_tile<DI>(kb, (kt + 1) * KT, N, base[(kt + 1) & 1], wave, lane);
    const LDS_AS uint16_t* tl = (const LDS_AS uint16_t*)kt_lds[kt & 1];
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
    // ReLU, head weight, sum over the heads: 8 of each token in the lane,
    // the other 8 in lane l ^ 32, which gets this lane's partial of the token
    // it stores and sends its own
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
        const float give = half ? p0 : p1, keep = half ? p1 : p0;
        const float sum = keep + __shfl_xor(give, 32, 64);
        const int key = kt * KT + rt * 32 + (lane & 31);
        if (tok[ct] < N && key <= tok[ct]) scores[(b * N + tok[ct]) * (int64_t)N + key] = sum;
      }
    }
  }
}

// ============================================================== token attention
// A 32-key chunk of kept tokens: its K rows in this wave's LDS tile (row-major,
// 16-byte chunks XOR-swizzled by kswz, read back as MFMA A operands) and its V
// rows in registers (lane owns 8 dims of a key group).
template <int D, int G>
struct GatherChunk {
  using C = DecCfg<D, G>;
  const LDS_AS uint16_t* kt;
  int lane;
  u32x4 vv[C::VPL];
  __device__ __forceinline__ u32x4 kfrag(int sb, int ks) const {
    const int row = sb * 16 + (lane & 15);
    const int c = (4 * ks + (lane >> 4)) ^ kswz<D>(row);
    return *reinterpret_cast<const LDS_AS u32x4*>(kt + row * D + c * 8);
  }
  __device__ __forceinline__ u32x4 vrow(int v) const { return vv[v]; }
  __device__ __forceinline__ float kscale(int, int) const { return 1.f; }
  __device__ __forceinline__ float vscale(int, int) const { return 1.f; }
};

// Waves per SIMD, as many as fit without spills: 128 VGPRs (four) for small
// groups, 168 (three) for four heads at d = 128, 256 (two) for eight heads.
template <int D, int G>
constexpr int token_attn_waves() { return G <= 2 || (G == 4 && D == 64) ? 4 : G == 4 ? 3 : 2; }

template <int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(token_attn_waves<D, G>())))
void token_attn_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                       const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
                       const int32_t* __restrict__ cnt, uint16_t* __restrict__ o, float* __restrict__ lse,
                       int Hkv, int N, int kmax, float scale_log2, int64_t n_waves) {
  using C = DecCfg<D, G>;
  constexpr int CH = D / 8, RPI = 64 / CH, NL = C::CK / RPI;  // lanes per row, rows per DMA, DMAs per chunk
  __shared__ __align__(1024) uint16_t ktile[4][C::CK * D];
  __shared__ float pbuf[4][C::CK][G];
  __shared__ float abuf[4][G];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
  const LDS_AS uint16_t* kt = (const LDS_AS uint16_t*)(ktile[wave]);
  const uint32_t kt_base = (uint32_t)(uintptr_t)kt;

  WaveAttn<D, G> wa;
  wa.init_rows(q + ((b * Hq + g * G) * (int64_t)N + t) * D, (int64_t)N * D);

  // kept positions base .. base + 63, one per lane; positions past nk repeat
  // the last kept token (a finite row whose weight the step masks to 0)
  auto ids = [&](int base) {
    const int p = min(base + lane, nk - 1);
    return min(max(row[p], 0), N - 1);
  };
  // chunk cc (0 or 1) of the 64 positions in iv.  K: each DMA brings RPI whole
  // rows (CH consecutive lanes per row, so every request covers full cache
  // lines), lane l landing in slot l of the tile; V: 16-byte pieces of rows.
  auto gather = [&](GatherChunk<D, G>& r, int iv, int cc) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int rr = i * RPI + lane / CH;
      const int key = __shfl(iv, 32 * cc + rr, 64);
      const int c = (lane % CH) ^ kswz<D>(rr);
      dma16(kb, (uint32_t)(key * D + c * 8) * 2u, __builtin_amdgcn_readfirstlane(kt_base + i * 1024));
    }
#pragma unroll
    for (int vi = 0; vi < C::VPL; ++vi) {
      const int key = __shfl(iv, 32 * cc + wa.pk + C::KGR * vi, 64);
      r.vv[vi] = *reinterpret_cast<const u32x4*>(vb + (int64_t)key * D + wa.pc * 8);
    }
  };

  // one 32-key chunk at a time (a second tile and register set would cost
  // more waves per SIMD than it hides)
  const int nch = (nk + C::CK - 1) / C::CK;
  GatherChunk<D, G> r;
  r.kt = kt;
  r.lane = lane;
  int iv = 0;
  for (int c = 0; c < nch; ++c) {
    if ((c & 1) == 0) iv = ids(c * C::CK);
    gather(r, iv, c & 1);
    wait_vm<C::VPL>();  // the K DMAs (issued before the V loads) have landed
    wa.step(r, c * C::CK, nk, scale_log2, pbuf[wave], abuf[wave]);
  }

  // sum the key groups: every lane of a dim slice ends with the totals
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = wa.acc[hh][e];
#pragma unroll
      for (int off = C::CHK; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
      wa.acc[hh][e] = x;
    }
  // O = acc / l (bf16), LSE = (m + log2 l) ln 2; head hh's state is in lane hh
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wa.l_run), hh));
    const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wa.m_run), hh));
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (wa.pk == 0) {
      u32x4 pkd;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2_t h2 = {(__bf16)(wa.acc[hh][2 * e] * inv), (__bf16)(wa.acc[hh][2 * e + 1] * inv)};
        pkd[e] = __builtin_bit_cast(uint32_t, h2);
      }
      *reinterpret_cast<u32x4*>(o + ((b * Hq + g * G + hh) * (int64_t)N + t) * D + wa.pc * 8) = pkd;
    }
    if (lse && lane == 0)
      lse[(b * Hq + g * G + hh) * (int64_t)N + t] = l > 0.f ? (m + __log2f(l)) * 0.6931471805599453f : -__builtin_inff();
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
