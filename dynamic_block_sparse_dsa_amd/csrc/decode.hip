// Single-token decode over a block-sparse KV cache.
//
// Method sources (by page and section):
//   "dynamic sparse attention explainer" (zblog.xzdbk.com/559.html),
//     "动态开销与计算收益的权衡": compute the index data when the cache is
//     written rather than reselecting from raw keys every step (the fp32 block
//     means of the key cache are built once, by dsa_kv_block_means);
//     "前沿方向": GQA/MQA share the KV cache and so one selection per group.
//   "稀疏注意力 vs Flash Attention v2" (pnsm.cn/news/1249548.html), section 1:
//     softmax of the scaled logits over the kept keys, times V.
//
// A step is four launches on the caller's stream:
//   1. decode_scores_kernel: score[j] = max over the group's heads of
//      (1/sqrt(d)) q_h . kbar_j, one 256-thread workgroup per 64 blocks of a
//      (sequence, KV head) unit -- a pure fp32 stream over the block means;
//   2. the shared top-k select, one row per unit (every row sees all blocks);
//   3. decode_attn_kernel: split-K over the kept blocks, one workgroup per
//      (unit, split), one kept block per wave at a time.  Q K^T uses
//      v_mfma_f32_16x16x32_bf16 with the key rows loaded straight from HBM as
//      the A operand and the group's query heads as B columns; P V is fp32
//      VALU over 16-byte V rows.  The workgroup writes its partial
//      (max, sum, acc[d]) per head;
//   4. decode_combine_kernel: merges the partials of each unit.
// The step is bound by HBM bandwidth: it must read the kept K/V blocks and
// the whole block-mean cache.
#include "dsa_internal.hpp"

namespace dsa {

constexpr int DEC_MAXG = 8;

// ============================================================== 1. scores
template <int D>
__global__ __launch_bounds__(256) void decode_scores_kernel(const uint16_t* __restrict__ q,
                                                            const float* __restrict__ kbar,
                                                            float* __restrict__ scores, int Hq, int Hkv, int nB,
                                                            float scale, int nchunks) {
  __shared__ f32x4 qs[DEC_MAXG][D / 4];
  const int G = Hq / Hkv;
  const int64_t unit = blockIdx.x / nchunks;
  const int chunk = blockIdx.x % nchunks;
  const int64_t s = unit / Hkv;
  const int g = (int)(unit % Hkv);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int e = t; e < G * D; e += 256) {
    const int hh = e / D, dd = e % D;
    const uint16_t raw = q[(s * Hq + g * G + hh) * (int64_t)D + dd];
    reinterpret_cast<float*>(&qs[hh][0])[dd] = __uint_as_float((uint32_t)raw << 16);
  }
  __syncthreads();
  const int blk = chunk * 64 + wave * 16 + (lane >> 2);
  const int quarter = lane & 3;
  float part[DEC_MAXG];
#pragma unroll
  for (int hh = 0; hh < DEC_MAXG; ++hh) part[hh] = 0.f;
  if (blk < nB) {
    const f32x4* krow = reinterpret_cast<const f32x4*>(kbar + (unit * nB + blk) * (int64_t)D);
#pragma unroll
    for (int m = 0; m < D / 16; ++m) {
      const int c = 4 * m + quarter;  // float4 chunk of the row
      const f32x4 kv = krow[c];
#pragma unroll
      for (int hh = 0; hh < DEC_MAXG; ++hh) {
        if (hh < G) {
          const f32x4 qv = qs[hh][c];
          part[hh] = __builtin_fmaf(kv[0], qv[0], part[hh]);
          part[hh] = __builtin_fmaf(kv[1], qv[1], part[hh]);
          part[hh] = __builtin_fmaf(kv[2], qv[2], part[hh]);
          part[hh] = __builtin_fmaf(kv[3], qv[3], part[hh]);
        }
      }
    }
  }
  float best = -__builtin_inff();
#pragma unroll
  for (int hh = 0; hh < DEC_MAXG; ++hh) {
    if (hh < G) {
      float v = part[hh];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      best = fmaxf(best, v * scale);
    }
  }
  if (quarter == 0 && blk < nB) scores[unit * nB + blk] = best;
}

// ============================================================== 3. split attention
template <int D, int BLK, int G>
struct DecCfg {
  static constexpr int WAVES = 4;
  static constexpr int CHK = D / 8;         // 16-byte chunks per row
  static constexpr int KGR = 64 / CHK;      // key groups in a wave for P V
  static constexpr int SUB = BLK / 16;      // 16-key MFMA subtiles per block
};

template <int D, int BLK, int G>
__global__ __launch_bounds__(256) void decode_attn_kernel(DecodeArgs a) {
  using C = DecCfg<D, BLK, G>;
  __shared__ float pbuf[C::WAVES][BLK][G];   // P of the wave's current block
  __shared__ float abuf[C::WAVES][G];        // rescale factor of the wave's heads
  __shared__ float mw[C::WAVES][G], lw[C::WAVES][G];
  __shared__ float accw[C::WAVES][G][D];

  const int unit = blockIdx.x / a.nsplit;
  const int split = blockIdx.x % a.nsplit;
  const int bps = (a.kmax + a.nsplit - 1) / a.nsplit;
  const int t0 = split * bps, t1 = min(a.kmax, t0 + bps);
  const int64_t s = unit / a.Hkv;
  const int g = unit % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = a.L;
  const uint16_t* kb = a.kc + (int64_t)unit * L * D;
  const uint16_t* vb = a.vc + (int64_t)unit * L * D;
  const int32_t* irow = a.idx + (int64_t)unit * a.kmax;
  const float NEG_INF = -__builtin_inff();

  // B operand: column n = lane % 16 is query head n of the group (zero past G),
  // slots 8 * (lane / 16) + e <-> dims ks * 32 + 8 * (lane / 16) + e
  const int n = lane & 15, lq = lane >> 4;
  u32x4 qf[D / 32];
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    qf[ks] = (u32x4){0, 0, 0, 0};
    if (n < G) qf[ks] = *reinterpret_cast<const u32x4*>(a.q + (s * a.Hq + g * G + n) * (int64_t)D + ks * 32 + 8 * lq);
  }

  float m_run = NEG_INF, l_run = 0.f;  // head n's state (lanes with n < G)
  // P V: lane owns dims 8 * (lane % CHK) .. +7 for keys lane / CHK + KGR * r
  const int pc = lane % C::CHK, pk = lane / C::CHK;
  float acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;

  for (int t = t0 + wave; t < t1; t += C::WAVES) {
    const int key0 = irow[t] * BLK;
    // ---- scores of the BLK keys for the G heads
    f32x4 sc[C::SUB];
#pragma unroll
    for (int sb = 0; sb < C::SUB; ++sb) {
      sc[sb] = (f32x4){0, 0, 0, 0};
      const int key = key0 + sb * 16 + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        u32x4 kf = (u32x4){0, 0, 0, 0};
        if (key < L) kf = *reinterpret_cast<const u32x4*>(kb + (int64_t)key * D + ks * 32 + 8 * lq);
        sc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf), as_bf16x8(qf[ks]), sc[sb], 0, 0, 0);
      }
    }
    // output: lane holds head column n, keys sb * 16 + 4 * lq + r
    float mloc = NEG_INF;
#pragma unroll
    for (int sb = 0; sb < C::SUB; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = key0 + sb * 16 + 4 * lq + r;
        const float x = (key < L) ? sc[sb][r] * a.scale_log2 : NEG_INF;
        sc[sb][r] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int sb = 0; sb < C::SUB; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(sc[sb][r] - m_run);
        lsum += p;
        if (n < G) pbuf[wave][sb * 16 + 4 * lq + r][n] = p;
      }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    l_run = l_run * alpha + lsum;
    if (lane < G) abuf[wave][lane] = alpha;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- acc = alpha * acc + P V
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float al = abuf[wave][hh];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= al;
    }
    for (int kk = pk; kk < BLK; kk += C::KGR) {
      const int key = key0 + kk;
      u32x4 vv = (u32x4){0, 0, 0, 0};
      if (key < L) vv = *reinterpret_cast<const u32x4*>(vb + (int64_t)key * D + pc * 8);
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16_lo(vv[e]);
        vf[2 * e + 1] = bf16_hi(vv[e]);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = pbuf[wave][kk][hh];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = __builtin_fmaf(p, vf[e], acc[hh][e]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- reduce the key groups of the wave, then merge the 4 waves
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = acc[hh][e];
      for (int off = C::CHK; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
      acc[hh][e] = v;
    }
  if (lane < G) {
    mw[wave][lane] = m_run;
    lw[wave][lane] = l_run;
  }
  if (pk == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) accw[wave][hh][pc * 8 + e] = acc[hh][e];
  }
  __syncthreads();
  for (int e = tid; e < G * (D + 2); e += 256) {
    const int hh = e / (D + 2), c = e % (D + 2);
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < C::WAVES; ++w) M = fmaxf(M, mw[w][hh]);
    float v = 0.f;
    if (c == 0) {
      v = M;
    } else {
#pragma unroll
      for (int w = 0; w < C::WAVES; ++w) {
        const float f = __builtin_amdgcn_exp2f(mw[w][hh] - M);  // 0 for a wave with no block
        v += f * (c == 1 ? lw[w][hh] : accw[w][hh][c - 2]);
      }
    }
    a.partial[(((int64_t)unit * a.nsplit + split) * G + hh) * (D + 2) + c] = v;
  }
}

// ============================================================== 4. combine
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ partial,
                                                             uint16_t* __restrict__ o, float* __restrict__ lse,
                                                             int Hq, int Hkv, int nsplit) {
  const int G = Hq / Hkv;
  const int unit = blockIdx.x;
  const int64_t s = unit / Hkv;
  const int g = unit % Hkv;
  for (int e = threadIdx.x; e < G * D; e += 256) {
    const int hh = e / D, dd = e % D;
    const float* p = partial + ((int64_t)unit * nsplit * G + hh) * (D + 2);
    const int stride = G * (D + 2);
    float M = -__builtin_inff();
    for (int c = 0; c < nsplit; ++c) M = fmaxf(M, p[c * stride]);
    float l = 0.f, v = 0.f;
    for (int c = 0; c < nsplit; ++c) {
      const float f = __builtin_amdgcn_exp2f(p[c * stride] - M);
      l += f * p[c * stride + 1];
      v += f * p[c * stride + 2 + dd];
    }
    const int64_t oh = s * Hq + g * G + hh;
    o[oh * D + dd] = (uint16_t)f32_to_bf16_rne(v / l);
    if (lse && dd == 0) lse[oh] = (M + __log2f(l)) * 0.69314718055994531f;
  }
}

// ============================================================== launch
int decode_splits(int S, int Hkv, int kmax) {
  const int64_t units = (int64_t)S * Hkv;
  if (units == 0 || kmax == 0) return 1;
  int64_t want = (2048 + units - 1) / units;  // aim for >= 2048 workgroups
  if (want < 1) want = 1;
  if (want > kmax) want = kmax;
  const int bps = (int)((kmax + want - 1) / want);
  return (kmax + bps - 1) / bps;  // every split gets at least one block
}

template <int D, int BLK>
static hipError_t launch_decode_attn(const DecodeArgs& a, hipStream_t stream) {
  const int G = a.Hq / a.Hkv;
  const dim3 grid((uint32_t)((int64_t)a.S * a.Hkv * a.nsplit)), blk(256);
  switch (G) {
    case 1: hipLaunchKernelGGL((decode_attn_kernel<D, BLK, 1>), grid, blk, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_attn_kernel<D, BLK, 2>), grid, blk, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_attn_kernel<D, BLK, 4>), grid, blk, 0, stream, a); break;
    case 8: hipLaunchKernelGGL((decode_attn_kernel<D, BLK, 8>), grid, blk, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int d, TopkParams p, hipStream_t stream) {
  const int64_t units = (int64_t)a.S * a.Hkv;
  if (units == 0) return hipSuccess;
  const int nchunks = (a.nB + 63) / 64;
  const dim3 g1((uint32_t)(units * nchunks)), b1(256);
  if (d == 64)
    hipLaunchKernelGGL(decode_scores_kernel<64>, g1, b1, 0, stream, a.q, a.kbar, a.scores, a.Hq, a.Hkv, a.nB,
                       a.scale, nchunks);
  else
    hipLaunchKernelGGL(decode_scores_kernel<128>, g1, b1, 0, stream, a.q, a.kbar, a.scores, a.Hq, a.Hkv, a.nB,
                       a.scale, nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_select_topk(a.scores, a.idx, nullptr, units, 1, a.nB, false, p, a.kmax, stream);
  if (e != hipSuccess) return e;
  if (d == 64)
    e = a.block == 64 ? launch_decode_attn<64, 64>(a, stream) : launch_decode_attn<64, 128>(a, stream);
  else
    e = a.block == 64 ? launch_decode_attn<128, 64>(a, stream) : launch_decode_attn<128, 128>(a, stream);
  if (e != hipSuccess) return e;
  if (d == 64)
    hipLaunchKernelGGL(decode_combine_kernel<64>, dim3((uint32_t)units), dim3(256), 0, stream, a.partial, a.o, a.lse,
                       a.Hq, a.Hkv, a.nsplit);
  else
    hipLaunchKernelGGL(decode_combine_kernel<128>, dim3((uint32_t)units), dim3(256), 0, stream, a.partial, a.o,
                       a.lse, a.Hq, a.Hkv, a.nsplit);
  return hipGetLastError();
}

}  // namespace dsa
