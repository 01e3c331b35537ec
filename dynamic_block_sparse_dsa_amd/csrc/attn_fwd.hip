// Sparse attention forward over the selected key blocks (bf16 MFMA, fp32
// online softmax).
//
// Method sources (by page and section):
//   "稀疏注意力 vs Flash Attention v2" (pnsm.cn/news/1249548.html), section 1:
//     the result is softmax(masked logits / sqrt(d_k)) times V; FlashAttention-2
//     tiles the work and keeps a running (incremental) softmax instead of the
//     full score matrix.
//   "dynamic sparse attention explainer" (zblog.xzdbk.com/559.html),
//     "硬件友好的稀疏计算实现" and "工程实践建议": block-sparse 64x64 or
//     128x128 tiles keep the kept work dense for the matrix units.
//   DeepSeek NSA article (pnsm.cn/news/1939904.html), section 2.2: the
//     weighted sum runs in bf16 (P is rounded to bf16 for the P V product).
//
// Design (gfx950):
//   * one workgroup per (batch, KV head, group of HG query heads, query block
//     i); wave w owns 32 query rows of one head, so the K/V tile of each kept
//     block is read from HBM/L2 once per workgroup and shared by its HG heads;
//   * K and V tiles go global -> LDS directly (global_load_lds_dwordx4: no
//     staging registers).  A wave instruction fills 1 KiB of LDS in lane
//     order, so each lane fetches the 16-byte chunk that an XOR swizzle
//     assigns to its LDS slot -- the swizzle spreads the MFMA operand reads
//     over all banks;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K rows are the A operand
//     (ds_read_b128), Q^T the B
//     operand (registers, for the whole workgroup).
//     One query row per lane (lanes l and l+32 hold the two key halves), so
//     the row max and sum are in-lane plus one cross-half exchange;
//   * O^T += V^T P^T: P leaves the S^T accumulators already in B-operand
//     order; the V^T A operand comes straight from the row-major V tile with
//     ds_read_b64_tr_b16 (within 16 lanes, lane i slot j receives element
//     i % 4 of the 8-byte chunk of source lane 4j + i / 4);
//   * LDS reads run ahead of the MFMAs that use them: K fragments four
//     k-steps ahead for 64-key tiles and one for 128-key tiles, the V^T
//     fragment of the next product one step ahead (without this the compiler
//     puts every read right before its MFMA and waits for it);
//   * the max is kept in raw logit units and 1/sqrt(d) * log2(e) is folded
//     into the single FMA that feeds exp2; the running max is only raised
//     (and O rescaled) when it grows by more than 8 (log2 units), which keeps
//     every P <= 256 and is exact after the final division;
//   * single K and V buffers, 4 barriers per tile: K(t+1) streams in while
//     the softmax and P V of tile t run, V(t+1) while Q K^T of tile t+1 runs;
//   * the diagonal block masks key > row by select; rows/keys past N read a
//     clamped (finite) row, are masked or discarded, never stored;
//   * workgroups are numbered XCD-aware (one head's query blocks share an
//     XCD's L2) and the heaviest (last) query blocks go first.
#include "attn_common.hpp"

namespace dsa {

template <int D, int BLK, int HG>
struct AttnCfg {
  static constexpr int SLABS = BLK / 32;  // 32-row slabs per head
  static constexpr int WAVES = HG * SLABS;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int CH = D / 8;                  // 16-byte chunks per row
  static constexpr int RPI = 1024 / (2 * D);        // rows per 1 KiB wave load
  static constexpr int LOADS = BLK * D * 2 / 1024;  // wave loads per tile (K or V)
  static constexpr int LOADS_PER_WAVE = LOADS / WAVES;
  static_assert(LOADS % WAVES == 0, "tile loads must split evenly over waves");
};

// Byte offset, relative to the first row of the tile, of the 16-byte chunk
// lane `lane` fetches for wave load n (row r, swizzled chunk c).
template <int D, int BLK, int HG>
__device__ __forceinline__ uint32_t tile_lane_offset(int n, int wave, int lane, bool v_swizzle, int* row_out) {
  using C = AttnCfg<D, BLK, HG>;
  const int inst = wave + n * C::WAVES;
  const int r = inst * C::RPI + lane / C::CH;
  const int c = (lane % C::CH) ^ (v_swizzle ? vswz<D>(r) : kswz<D>(r));
  *row_out = r;
  return (uint32_t)(r * D + c * 8) * 2u;
}

// Enqueue this wave's share of one K or V tile (rows key0 .. key0+BLK-1).
// off[n] are the precomputed lane offsets; a full tile only moves the
// scalar base, a ragged last tile clamps each row to N-1.
template <int D, int BLK, int HG>
__device__ __forceinline__ void issue_tile(const uint16_t* g, uint32_t lds_base, const uint32_t* off, int key0, int N,
                                           int wave, int lane, bool v_swizzle) {
  using C = AttnCfg<D, BLK, HG>;
  if (key0 + BLK <= N) {
    const uint16_t* base = g + (int64_t)key0 * D;
#pragma unroll
    for (int n = 0; n < C::LOADS_PER_WAVE; ++n)
      dma16(base, off[n], __builtin_amdgcn_readfirstlane(lds_base + (wave + n * C::WAVES) * 1024));
  } else {
#pragma unroll
    for (int n = 0; n < C::LOADS_PER_WAVE; ++n) {
      int r;
      const uint32_t o = tile_lane_offset<D, BLK, HG>(n, wave, lane, v_swizzle, &r);
      const int key = min(key0 + r, N - 1);
      const uint32_t clamped = o - (uint32_t)(r * D * 2) + (uint32_t)(key * D * 2);
      dma16(g, clamped, __builtin_amdgcn_readfirstlane(lds_base + (wave + n * C::WAVES) * 1024));
    }
  }
}

// NB = 1: single K and V buffers, four barriers per tile (K(t+1) streams in
// while the softmax and P V of tile t run, V(t+1) while Q K^T of tile t+1
// runs).  NB = 2: two of each, one barrier per tile (K(t+1) and V(t+1) go to
// the other buffers while tile t runs), where the LDS holds them without
// costing a workgroup per CU.
template <int D, int BLK, int HG, int NB>
__device__ __forceinline__ void attn_body(const AttnArgs& a, LDS_AS uint16_t* ks_all, LDS_AS uint16_t* vs_all) {
  using C = AttnCfg<D, BLK, HG>;
  constexpr int NV = C::LOADS_PER_WAVE;  // loads per wave per tile (K or V)

  const int G = a.Hq / a.Hkv;
  const int hchunks = G / HG;
  const uint32_t L = xcd_logical_id(blockIdx.x, gridDim.x);
  const int i = a.nB - 1 - (int)(L % (uint32_t)a.nB);
  const uint32_t u = L / (uint32_t)a.nB;
  const int hc = (int)(u % (uint32_t)hchunks);
  const int64_t bg = u / (uint32_t)hchunks;  // b * Hkv + g
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

  const uint16_t* qh = a.q + (b * a.Hq + h) * (int64_t)N * D;
  const uint16_t* kgp = a.k + bg * (int64_t)N * D;
  const uint16_t* vgp = a.v + bg * (int64_t)N * D;
  // the index row is read through the constant address space: uniform scalar
  // loads, counted by lgkmcnt, so they never wait on the tile DMA (vmcnt)
  const CONST_AS int32_t* irow = (const CONST_AS int32_t*)(a.idx + (bg * a.nB + i) * (int64_t)a.kmax);
  // counts and block ids are clamped into range: an index array that did not
  // come from a selection call gives wrong results, never an access outside
  // the tensors
  const int n_sel = min(max(((const CONST_AS int32_t*)a.cnt)[bg * a.nB + i], 0), a.kmax);
  auto blk_at = [&](int t) { return min(max(irow[t], 0), a.nB - 1); };
  const uint32_t ks_base0 = (uint32_t)(uintptr_t)ks_all, vs_base0 = (uint32_t)(uintptr_t)vs_all;
  constexpr uint32_t TILE_BYTES = BLK * D * 2;

  uint32_t koff[C::LOADS_PER_WAVE], voff[C::LOADS_PER_WAVE];
#pragma unroll
  for (int n = 0; n < C::LOADS_PER_WAVE; ++n) {
    int r;
    koff[n] = tile_lane_offset<D, BLK, HG>(n, wave, lane, false, &r);
    voff[n] = tile_lane_offset<D, BLK, HG>(n, wave, lane, true, &r);
  }

  if (n_sel > 0) {
    const int j0 = blk_at(0);
    issue_tile<D, BLK, HG>(kgp, ks_base0, koff, j0 * BLK, N, wave, lane, false);
    issue_tile<D, BLK, HG>(vgp, vs_base0, voff, j0 * BLK, N, wave, lane, true);
  }

  // Q^T fragments (B operand): lane holds its row, dims ks*16 + 8*half .. +7.
  // The empty asm "uses" them here so the compiler's waits for these loads
  // land before the loop (where they would otherwise also wait on the DMA).
  u32x4 qf[D / 16];
  {
    const uint16_t* qr = qh + (int64_t)min(row, N - 1) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qr + ks * 16);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = (f32x16){};
  const float NEG_INF = -__builtin_inff();
  const float c2 = a.scale_log2;  // log2(e) / sqrt(d)
  float m_run = NEG_INF;          // running max of raw logits, same in lanes l and l^32
  float l_part = 0.f;             // this lane's share of the row sum

  for (int t = 0; t < n_sel; ++t) {
    const int j = blk_at(t);
    const bool diag = (j == i);
    const bool more = t + 1 < n_sel;
    const int jn = more ? blk_at(t + 1) : 0;
    const int buf = NB == 2 ? (t & 1) : 0;
    const LDS_AS uint16_t* ks_l = ks_all + buf * (BLK * D);
    const LDS_AS uint16_t* vs_l = vs_all + buf * (BLK * D);

    if constexpr (NB == 2) {
      // ---- K(t), V(t) resident; every wave is done with tile t - 1, whose
      // buffers take K(t+1), V(t+1) now
      wait_vm<0>();
      __syncthreads();
      if (more) {
        const uint32_t nb = (uint32_t)(buf ^ 1) * TILE_BYTES;
        issue_tile<D, BLK, HG>(kgp, ks_base0 + nb, koff, jn * BLK, N, wave, lane, false);
        issue_tile<D, BLK, HG>(vgp, vs_base0 + nb, voff, jn * BLK, N, wave, lane, true);
      }
    } else {
      // ---- K(t) resident (V(t) may still be in flight; Q loads are older)
      wait_vm<NV>();
      __syncthreads();
    }
    f32x16 s[BLK / 32];
#pragma unroll
    for (int st = 0; st < BLK / 32; ++st) s[st] = (f32x16){};
    {
      // K fragments are read KLOOK k-steps ahead of the MFMAs that use them
      // (LDS latency exceeds two MFMAs); the scheduling barriers keep the
      // compiler from sinking each read next to its use.  128-key tiles
      // (four MFMAs per k-step) have registers for one step.
      constexpr int NKS = D / 16, NST = BLK / 32;
      constexpr int KLOOK = BLK == 64 ? 4 : 1;
      auto kread = [&](int ks, u32x4* dst) {
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const int kr = st * 32 + (lane & 31);
          const int c = (2 * ks + half) ^ kswz<D>(kr);
          dst[st] = *reinterpret_cast<const LDS_AS u32x4*>(ks_l + kr * D + c * 8);
        }
      };
      u32x4 kb[KLOOK + 1][NST];
#pragma unroll
      for (int p = 0; p < KLOOK && p < NKS; ++p) kread(p, kb[p]);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (KLOOK == 0) kread(ks, kb[0]);
        else if (ks + KLOOK < NKS) kread(ks + KLOOK, kb[(ks + KLOOK) % (KLOOK + 1)]);
        if (KLOOK > 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < NST; ++st)
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kb[ks % (KLOOK + 1)][st]), as_bf16x8(qf[ks]),
                                                          s[st], 0, 0, 0);
        if (KLOOK > 0) __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (NB == 1) {
      __syncthreads();  // every wave is done reading K(t)
      if (more) issue_tile<D, BLK, HG>(kgp, ks_base0, koff, jn * BLK, N, wave, lane, false);
    }

    // ---- causal mask on the diagonal block, row max (raw units)
    if (diag) {
#pragma unroll
      for (int st = 0; st < BLK / 32; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key_in_blk = st * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          s[st][r] = (key_in_blk > row_in_blk) ? NEG_INF : s[st][r];
        }
    }
    float mloc = NEG_INF;
#pragma unroll
    for (int st = 0; st < BLK / 32; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[st][r]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    if (__any((m_new - m_run) * c2 > 8.0f)) {
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
      l_part *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c2;
    // ---- P = exp2(s * c2 - m * c2), packed to bf16 in B-operand order
    u32x4 pf[BLK / 16];
#pragma unroll
    for (int kk = 0; kk < BLK / 16; ++kk) {
      const int st = kk >> 1, rb = 8 * (kk & 1);
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st][rb + e], c2, -mc));
        l_part += p[e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2_t pk = {(__bf16)p[2 * e], (__bf16)p[2 * e + 1]};
        pf[kk][e] = __builtin_bit_cast(uint32_t, pk);
      }
    }

    // ---- V(t) resident (K(t+1) may be in flight)
    if constexpr (NB == 1) {
      if (more) wait_vm<NV>(); else wait_vm<0>();
      __syncthreads();
    }
    // ---- O^T += V^T P^T, A operand by transposed LDS reads: the (d-tile,
    // key-step) products in one sequence with the next step's V^T fragment in
    // flight (the scheduling barriers keep each read a step ahead of its use)
    {
      constexpr int KK = BLK / 16, NPV = (D / 32) * KK;
      const int grp = (lane >> 4) & 1, si = lane & 15;  // 16-lane group within the half; source index
      auto vread = [&](int step, u32x4& vf) {
        const int dt = step / KK, kk = step % KK;
        const int d = dt * 32 + 16 * grp + 4 * (si & 3);
        const int cbase = d >> 3, sub = (d & 7) * 2;  // 16-byte chunk and byte offset (0 or 8)
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) {
          const int key = 16 * kk + 8 * sg + 4 * half + (si >> 2);
          const int c = cbase ^ vswz<D>(key);
          const LDS_AS char* addr = reinterpret_cast<const LDS_AS char*>(vs_l + key * D + c * 8) + sub;
          const i16x4 v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)addr);
          const u32x2 w = __builtin_bit_cast(u32x2, v4);
          vf[2 * sg] = w[0];
          vf[2 * sg + 1] = w[1];
        }
      };
      u32x4 vb[2];
      vread(0, vb[0]);
#pragma unroll
      for (int step = 0; step < NPV; ++step) {
        if (step + 1 < NPV) vread(step + 1, vb[(step + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        oacc[step / KK] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vb[step & 1]), as_bf16x8(pf[step % KK]),
                                                                 oacc[step / KK], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (NB == 1) {
      __syncthreads();  // every wave is done reading V(t)
      if (more) issue_tile<D, BLK, HG>(vgp, vs_base0, voff, jn * BLK, N, wave, lane, true);
    }
  }

  // ---- epilogue: O = acc / l (bf16), LSE = ln(sum) + max
  const float l_tot = l_part + __shfl_xor(l_part, 32, 64);
  if (row < N) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = a.o + ((b * a.Hq + h) * (int64_t)N + row) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const bf16x2_t lo = {(__bf16)(oacc[dt][4 * q4 + 0] * inv), (__bf16)(oacc[dt][4 * q4 + 1] * inv)};
        const bf16x2_t hi = {(__bf16)(oacc[dt][4 * q4 + 2] * inv), (__bf16)(oacc[dt][4 * q4 + 3] * inv)};
        u32x2 w;
        w[0] = __builtin_bit_cast(uint32_t, lo);
        w[1] = __builtin_bit_cast(uint32_t, hi);
        *reinterpret_cast<u32x2*>(orow + dt * 32 + 8 * q4 + 4 * half) = w;
      }
    }
    if (a.lse && half == 0)
      a.lse[(b * a.Hq + h) * (int64_t)N + row] = (m_run * c2 + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

template <int D, int BLK, int HG, int NB>
__global__ __launch_bounds__((AttnCfg<D, BLK, HG>::THREADS)) __attribute__((amdgpu_waves_per_eu(2)))
void sparse_attn_fwd_kernel(AttnArgs a) {
  __shared__ __align__(1024) uint16_t Ks[NB][BLK * D];
  __shared__ __align__(1024) uint16_t Vs[NB][BLK * D];
  attn_body<D, BLK, HG, NB>(a, (LDS_AS uint16_t*)(Ks[0]), (LDS_AS uint16_t*)(Vs[0]));
}

// Double buffers where they cost no workgroup per CU: a workgroup of 8 waves
// (two per SIMD) is alone on its CU anyway, and 4-wave workgroups of 64-key
// tiles still fit two per CU with 64 KiB each.
template <int D, int BLK, int HG>
constexpr int attn_buffers() { return AttnCfg<D, BLK, HG>::WAVES >= 4 && 2 * 2 * BLK * D * 2 <= 80 * 1024 ? 2 : AttnCfg<D, BLK, HG>::WAVES == 8 ? 2 : 1; }

template <int D, int BLK, int HG>
static hipError_t launch_attn_cfg(const AttnArgs& a, hipStream_t stream) {
  using C = AttnCfg<D, BLK, HG>;
  const int G = a.Hq / a.Hkv;
  const int64_t n_wg = (int64_t)a.B * a.Hkv * (G / HG) * a.nB;
  if (n_wg == 0) return hipSuccess;
  constexpr int NB = attn_buffers<D, BLK, HG>();
  hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BLK, HG, NB>), dim3((uint32_t)n_wg), dim3(C::THREADS), 0, stream, a);
  return hipGetLastError();
}

template <int D, int BLK>
static hipError_t launch_attn_d_blk(const AttnArgs& a, hipStream_t stream) {
  // heads per workgroup: as many of the group as fit in 256 query rows
  const int G = a.Hq / a.Hkv;
  if constexpr (BLK == 64) {
    if (G % 4 == 0) return launch_attn_cfg<D, BLK, 4>(a, stream);
    if (G % 2 == 0) return launch_attn_cfg<D, BLK, 2>(a, stream);
    return launch_attn_cfg<D, BLK, 1>(a, stream);
  } else {
    if (G % 2 == 0) return launch_attn_cfg<D, BLK, 2>(a, stream);
    return launch_attn_cfg<D, BLK, 1>(a, stream);
  }
}

hipError_t launch_sparse_attn_fwd(const AttnArgs& a, int d, int block, hipStream_t stream) {
  if (d == 64) return block == 64 ? launch_attn_d_blk<64, 64>(a, stream) : launch_attn_d_blk<64, 128>(a, stream);
  return block == 64 ? launch_attn_d_blk<128, 64>(a, stream) : launch_attn_d_blk<128, 128>(a, stream);
}

}  // namespace dsa
