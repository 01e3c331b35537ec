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
//     i); wave w owns 32 query rows of one head; the K/V tile of each kept
//     block is loaded once per workgroup and shared by all HG heads;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: K rows are the A operand
//     (read from LDS), Q^T the B operand (kept in registers for the whole
//     workgroup).  The output puts one query row in each lane (lanes l and
//     l+32 hold the two halves of the keys), so the softmax row reductions
//     are in-lane plus one cross-half exchange;
//   * O^T += V^T P^T: P leaves the S^T accumulators already in B-operand
//     order; V is written to LDS transposed ([d][key]) so its A operand is two
//     8-byte reads;
//   * exp2 with log2(e)/sqrt(d) folded into one multiply; the running max is
//     only raised (and O rescaled) when it grows by more than 2^8, which keeps
//     every P <= 256 and is exact after the final division;
//   * the diagonal block masks key > row by select (never by adding -inf to
//     a value), and rows/keys past N are zero-filled, so no garbage can reach
//     an output;
//   * workgroups are numbered XCD-aware (one head's query blocks share an
//     XCD's L2) and the heaviest (last) query blocks go first.
#include <mutex>

#include "dsa_internal.hpp"

namespace dsa {

template <int D, int BLK, int HG>
struct AttnCfg {
  static constexpr int SLABS = BLK / 32;  // 32-row slabs per head
  static constexpr int WAVES = HG * SLABS;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KP = D + 8;    // K tile pitch in LDS (elements): 16 B pad
  static constexpr int VP = BLK + 4;  // V^T tile pitch in LDS (elements): 8 B pad
  static constexpr int K_CHUNKS = BLK * D / 8;         // 16-byte chunks of a K tile
  static constexpr int V_PATCHES = (BLK / 4) * (D / 8);  // 4 keys x 8 dims patches
  static constexpr int K_PER_T = (K_CHUNKS + THREADS - 1) / THREADS;
  static constexpr int V_PER_T = (V_PATCHES + THREADS - 1) / THREADS;
  static constexpr int LDS_BYTES = (BLK * KP + D * VP) * 2;
};

__device__ __forceinline__ uint32_t half_of(u32x4 w, int e) {
  // 16-bit element e (0..7) of an 8 x bf16 vector
  const uint32_t word = w[e >> 1];
  return (e & 1) ? (word >> 16) : (word & 0xffffu);
}

template <int D, int BLK, int HG>
__global__ __launch_bounds__((AttnCfg<D, BLK, HG>::THREADS)) void sparse_attn_fwd_kernel(AttnArgs a) {
  using C = AttnCfg<D, BLK, HG>;
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* Ks = lds;                 // [BLK][KP]   key-major
  uint16_t* Vt = lds + BLK * C::KP;   // [D][VP]     dim-major (transposed)

  const int G = a.Hq / a.Hkv;
  const int hchunks = G / HG;
  const uint32_t L = xcd_logical_id(blockIdx.x, gridDim.x);
  const int i = a.nB - 1 - (int)(L % (uint32_t)a.nB);
  const uint32_t u = L / (uint32_t)a.nB;
  const int hc = (int)(u % (uint32_t)hchunks);
  const int64_t bg = u / (uint32_t)hchunks;  // b * Hkv + g
  const int64_t b = bg / a.Hkv;
  const int g = (int)(bg % a.Hkv);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = wave / C::SLABS, slab = wave % C::SLABS;
  const int h = g * G + hc * HG + hl;
  const int half = lane >> 5;
  const int row_in_blk = slab * 32 + (lane & 31);
  const int row = i * BLK + row_in_blk;
  const int N = a.N;

  const uint16_t* qh = a.q + (b * a.Hq + h) * (int64_t)N * D;
  const uint16_t* kgp = a.k + bg * (int64_t)N * D;
  const uint16_t* vgp = a.v + bg * (int64_t)N * D;
  const int32_t* irow = a.idx + (bg * a.nB + i) * (int64_t)a.kmax;
  const int n_sel = a.cnt[bg * a.nB + i];

  // Q^T fragments: lane holds its row, dims ks*16 + 8*half .. +7
  u32x4 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    qf[ks] = (u32x4){0, 0, 0, 0};
    if (row < N) qf[ks] = *reinterpret_cast<const u32x4*>(qh + (int64_t)row * D + ks * 16 + 8 * half);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = (f32x16){};
  const float NEG_INF = -__builtin_inff();
  float m_run = NEG_INF;  // running max (log2 domain), same in lanes l and l^32
  float l_part = 0.f;     // this lane's share of the row sum

  u32x4 kst[C::K_PER_T];
  u32x4 vst[C::V_PER_T][4];

  auto load_tile = [&](int j) {
    const int key0 = j * BLK;
#pragma unroll
    for (int n = 0; n < C::K_PER_T; ++n) {
      const int c = tid + n * C::THREADS;
      kst[n] = (u32x4){0, 0, 0, 0};
      if (c < C::K_CHUNKS) {
        const int r = c / (D / 8), col = c % (D / 8);
        if (key0 + r < N) kst[n] = *reinterpret_cast<const u32x4*>(kgp + (int64_t)(key0 + r) * D + col * 8);
      }
    }
#pragma unroll
    for (int n = 0; n < C::V_PER_T; ++n) {
      const int p = tid + n * C::THREADS;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) vst[n][rr] = (u32x4){0, 0, 0, 0};
      if (p < C::V_PATCHES) {
        const int kq = p / (D / 8), dg = p % (D / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key = key0 + 4 * kq + rr;
          if (key < N) vst[n][rr] = *reinterpret_cast<const u32x4*>(vgp + (int64_t)key * D + dg * 8);
        }
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int n = 0; n < C::K_PER_T; ++n) {
      const int c = tid + n * C::THREADS;
      if (c < C::K_CHUNKS) {
        const int r = c / (D / 8), col = c % (D / 8);
        *reinterpret_cast<u32x4*>(Ks + r * C::KP + col * 8) = kst[n];
      }
    }
#pragma unroll
    for (int n = 0; n < C::V_PER_T; ++n) {
      const int p = tid + n * C::THREADS;
      if (p < C::V_PATCHES) {
        const int kq = p / (D / 8), dg = p % (D / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          u32x2 w;
          w[0] = half_of(vst[n][0], e) | (half_of(vst[n][1], e) << 16);
          w[1] = half_of(vst[n][2], e) | (half_of(vst[n][3], e) << 16);
          *reinterpret_cast<u32x2*>(Vt + (dg * 8 + e) * C::VP + 4 * kq) = w;
        }
      }
    }
  };

  if (n_sel > 0) load_tile(irow[0]);
  for (int t = 0; t < n_sel; ++t) {
    const int j = irow[t];
    __syncthreads();  // every wave is done with the previous tile
    store_tile();
    __syncthreads();
    if (t + 1 < n_sel) load_tile(irow[t + 1]);  // in flight during the math below
    const bool diag = (j == i);

#pragma unroll
    for (int hb = 0; hb < BLK / 64; ++hb) {
      // ---- S^T = K Q^T for keys hb*64 .. hb*64+63 (two 32-key subtiles)
      f32x16 s[2] = {(f32x16){}, (f32x16){}};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 kf =
              *reinterpret_cast<const u32x4*>(Ks + (hb * 64 + st * 32 + (lane & 31)) * C::KP + ks * 16 + 8 * half);
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[ks]), s[st], 0, 0, 0);
        }
      }
      // ---- scale, causal mask on the diagonal block, row max
      float mloc = NEG_INF;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[st][r] * a.scale_log2;
          if (diag) {
            const int key_in_blk = hb * 64 + st * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            x = (key_in_blk > row_in_blk) ? NEG_INF : x;
          }
          s[st][r] = x;
          mloc = fmaxf(mloc, x);
        }
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
      const float m_new = fmaxf(m_run, mloc);
      if (__any(m_new > m_run + 8.0f)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
        l_part *= alpha;
        m_run = m_new;
      }
      // ---- P = exp2(S - m), packed to bf16 in B-operand order
      u32x4 pf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int st = kk >> 1, rb = 8 * (kk & 1);
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(s[st][rb + e] - m_run);
          l_part += p[e];
        }
        pf[kk] = (u32x4){pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                         pack_bf16x2(p[6], p[7])};
      }
      // ---- O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const uint16_t* vr = Vt + (dt * 32 + (lane & 31)) * C::VP + hb * 64 + kk * 16 + 4 * half;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
          const u32x4 vf = (u32x4){lo[0], lo[1], hi[0], hi[1]};
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[kk]), oacc[dt], 0, 0, 0);
        }
      }
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
        u32x2 w;
        w[0] = pack_bf16x2(oacc[dt][4 * q4 + 0] * inv, oacc[dt][4 * q4 + 1] * inv);
        w[1] = pack_bf16x2(oacc[dt][4 * q4 + 2] * inv, oacc[dt][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + dt * 32 + 8 * q4 + 4 * half) = w;
      }
    }
    if (a.lse && half == 0) a.lse[(b * a.Hq + h) * (int64_t)N + row] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
  }
}

template <int D, int BLK, int HG>
static hipError_t launch_attn_cfg(const AttnArgs& a, hipStream_t stream) {
  using C = AttnCfg<D, BLK, HG>;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&sparse_attn_fwd_kernel<D, BLK, HG>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
  });
  if (attr_err != hipSuccess) return attr_err;
  const int G = a.Hq / a.Hkv;
  const int64_t n_wg = (int64_t)a.B * a.Hkv * (G / HG) * a.nB;
  if (n_wg == 0) return hipSuccess;
  hipLaunchKernelGGL((sparse_attn_fwd_kernel<D, BLK, HG>), dim3((uint32_t)n_wg), dim3(C::THREADS), C::LDS_BYTES,
                     stream, a);
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
