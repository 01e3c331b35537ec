// Pieces of the decode attention shared by the contiguous-cache kernels
// (decode.hip) and the paged-cache kernel (decode_paged.hip): DPP group sums
// and one wave's online-softmax attention over 32-key chunks (WaveAttn).
#pragma once

#include "dsa_internal.hpp"

namespace dsa {

// sum over aligned groups of W = 8 or 16 lanes, in every lane of the group
// (DPP: two quad permutes, then the half-row and row mirrors)
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half mirror
  if (W == 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// Block-mean scans: the TPR = D/8 lanes of a row group hold dims 4c .. 4c+3
// and D/2 + 4c .. + 3 (c = lane % TPR), so each 16-byte-per-lane load covers
// whole 256-byte stretches of a row (full cache lines).  qv[0..3] and
// qv[4..7] are this lane's query values for those dims.
template <int D>
__device__ __forceinline__ void load_q_halves(const uint16_t* qrow, int c, float (&qv)[8]) {
  const u32x2 w0 = *reinterpret_cast<const u32x2*>(qrow + 4 * c);
  const u32x2 w1 = *reinterpret_cast<const u32x2*>(qrow + D / 2 + 4 * c);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    qv[2 * e] = bf16_lo(w0[e]);
    qv[2 * e + 1] = bf16_hi(w0[e]);
    qv[4 + 2 * e] = bf16_lo(w1[e]);
    qv[4 + 2 * e + 1] = bf16_hi(w1[e]);
  }
}

// Work unit of a wave: a 32-key chunk of a kept block.
template <int D, int G>
struct DecCfg {
  static constexpr int CK = 32;           // keys per chunk
  static constexpr int CHK = D / 8;       // 16-byte pieces per row
  static constexpr int KGR = 64 / CHK;    // key groups in a wave for P V
  static constexpr int SUB = CK / 16;     // 16-key MFMA subtiles per chunk
  static constexpr int VPL = CK / KGR;    // V rows per lane
};

// the loaded K (MFMA A operands) and V rows of one chunk
template <int D, int G>
struct ChunkRegs {
  using C = DecCfg<D, G>;
  u32x4 kf[C::SUB][D / 32];
  u32x4 vv[C::VPL];
  __device__ __forceinline__ u32x4 kfrag(int sb, int ks) const { return kf[sb][ks]; }
  __device__ __forceinline__ u32x4 vrow(int v) const { return vv[v]; }
  __device__ __forceinline__ float kscale(int, int) const { return 1.f; }
  __device__ __forceinline__ float vscale(int, int) const { return 1.f; }
};

// 8 E4M3 codes (OCP) -> 8 bf16, exactly (every E4M3 value is a bf16 value)
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 w) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    r[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.0f, false));
    r[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.0f, true));
  }
  return r;
}

// The same chunk from an FP8 cache: the codes (half the bytes of bf16) and
// the fp32 row scales of the keys this lane's scores cover (keys sb * 16 +
// 4 (lane / 16) + j).  Codes become bf16 MFMA operands as they are used; the
// K scale multiplies the key's logit and the V scale its softmax weight.
template <int D, int G>
struct ChunkRegs8 {
  using C = DecCfg<D, G>;
  u32x2 kf[C::SUB][D / 32];
  u32x2 vv[C::VPL];
  f32x4 ks[C::SUB], vs[C::SUB];
  __device__ __forceinline__ u32x4 kfrag(int sb, int k) const { return fp8x8_to_bf16x8(kf[sb][k]); }
  __device__ __forceinline__ u32x4 vrow(int v) const { return fp8x8_to_bf16x8(vv[v]); }
  __device__ __forceinline__ float kscale(int sb, int j) const { return ks[sb][j]; }
  __device__ __forceinline__ float vscale(int sb, int j) const { return vs[sb][j]; }
};

// One wave's online-softmax state for the G query heads of a unit, and the
// per-chunk work.  Q K^T on v_mfma_f32_16x16x32_bf16 (key rows as the A
// operand, heads as B columns); P goes through a per-wave LDS row to the
// P V layout (lane owns 8 dims of a key group), P V in fp32 VALU.
template <int D, int G>
struct WaveAttn {
  using C = DecCfg<D, G>;
  u32x4 qf[D / 32];
  float m_run, l_run;  // head n's state (lanes with n < G)
  float acc[G][8];
  int lane, n, lq, pc, pk;

  __device__ __forceinline__ void init(const DecodeArgs& a, int64_t s, int g) { init(a.q, a.Hq, s, g); }

  // q [S, Hq, D]: the group's heads of sequence s
  __device__ __forceinline__ void init(const uint16_t* q, int Hq, int64_t s, int g) {
    init_rows(q + (s * Hq + g * G) * (int64_t)D, D);
  }

  // query row of the group's head hh at q0 + hh * head_stride
  __device__ __forceinline__ void init_rows(const uint16_t* q0, int64_t head_stride) {
    lane = threadIdx.x & 63;
    n = lane & 15;
    lq = lane >> 4;
    pc = lane % C::CHK;
    pk = lane / C::CHK;
    // B operand: column n = lane % 16 is query head n of the group (zero past
    // G), slots 8 * (lane / 16) + e <-> dims ks * 32 + 8 * (lane / 16) + e
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      qf[ks] = (u32x4){0, 0, 0, 0};
      if (n < G)
        qf[ks] = *reinterpret_cast<const u32x4*>(q0 + n * head_stride + ks * 32 + 8 * lq);
    }
    m_run = -__builtin_inff();
    l_run = 0.f;
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
  }

  // issue every load of the chunk starting at key0 (keys clamped to L-1)
  __device__ __forceinline__ void load(ChunkRegs<D, G>& r, const uint16_t* kb, const uint16_t* vb, int key0,
                                       int L) const {
#pragma unroll
    for (int sb = 0; sb < C::SUB; ++sb) {
      const int key = min(key0 + sb * 16 + (lane & 15), L - 1);
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        r.kf[sb][ks] =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (int64_t)key * D + ks * 32 + 8 * lq));
    }
#pragma unroll
    for (int v = 0; v < C::VPL; ++v) {
      const int key = min(key0 + pk + C::KGR * v, L - 1);
      r.vv[v] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + (int64_t)key * D + pc * 8));
    }
  }

  // fold the chunk into the state; pbuf / abuf are this wave's LDS rows
  // the FP8 chunk: codes and the row scales of this lane's keys (ksb, vsb
  // are the tile's BLK scales); scales of keys past L are 0
  __device__ __forceinline__ void load8(ChunkRegs8<D, G>& r, const uint8_t* kb, const uint8_t* vb, const float* ksb,
                                        const float* vsb, int key0, int L) const {
#pragma unroll
    for (int sb = 0; sb < C::SUB; ++sb) {
      const int key = min(key0 + sb * 16 + (lane & 15), L - 1);
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        r.kf[sb][ks] =
            __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(kb + (int64_t)key * D + ks * 32 + 8 * lq));
    }
#pragma unroll
    for (int v = 0; v < C::VPL; ++v) {
      const int key = min(key0 + pk + C::KGR * v, L - 1);
      r.vv[v] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vb + (int64_t)key * D + pc * 8));
    }
#pragma unroll
    for (int sb = 0; sb < C::SUB; ++sb) {
      const int k0 = key0 + sb * 16 + 4 * lq;  // 4 consecutive keys, 16-byte aligned in the tile
      const f32x4 kv = *reinterpret_cast<const f32x4*>(ksb + k0);
      const f32x4 vv = *reinterpret_cast<const f32x4*>(vsb + k0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r.ks[sb][j] = k0 + j < L ? kv[j] : 0.f;
        r.vs[sb][j] = k0 + j < L ? vv[j] : 0.f;
      }
    }
  }

  template <class Regs>
  __device__ __forceinline__ void step(const Regs& r, int key0, int L, float scale_log2, float (*pbuf)[G],
                                       float* abuf) {
    const float NEG_INF = -__builtin_inff();
    f32x4 sc[C::SUB];
#pragma unroll
    for (int sb = 0; sb < C::SUB; ++sb) {
      sc[sb] = (f32x4){0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        sc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r.kfrag(sb, ks)), as_bf16x8(qf[ks]), sc[sb], 0, 0, 0);
    }
    // output: lane holds head column n, keys sb * 16 + 4 * lq + j (keys past L masked)
    float mloc = NEG_INF;
#pragma unroll
    for (int sb = 0; sb < C::SUB; ++sb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = key0 + sb * 16 + 4 * lq + j;
        const float x = (key < L) ? sc[sb][j] * r.kscale(sb, j) * scale_log2 : NEG_INF;
        sc[sb][j] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);  // finite: a chunk holds a key below L
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int sb = 0; sb < C::SUB; ++sb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pv = __builtin_amdgcn_exp2f(sc[sb][j] - m_run);
        lsum += pv;
        if (n < G) pbuf[sb * 16 + 4 * lq + j][n] = pv * r.vscale(sb, j);  // V scale folded into the weight
      }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    l_run = l_run * alpha + lsum;
    if (lane < G) abuf[lane] = alpha;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- acc = alpha * acc + P V
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float al = abuf[hh];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= al;
    }
#pragma unroll
    for (int v = 0; v < C::VPL; ++v) {
      const int kk = pk + C::KGR * v;
      const u32x4 vr = r.vrow(v);
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16_lo(vr[e]);
        vf[2 * e + 1] = bf16_hi(vr[e]);
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pw = pbuf[kk][hh];  // 0 for keys past L
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = __builtin_fmaf(pw, vf[e], acc[hh][e]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // reduce the wave's key groups and leave (max, sum, acc[d]) per head in LDS
  __device__ __forceinline__ void to_lds(float* mw, float* lw, float (*accw)[D]) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[hh][e];
#pragma unroll
        for (int off = C::CHK; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
        acc[hh][e] = v;
      }
    if (lane < G) {
      mw[lane] = m_run;
      lw[lane] = l_run;
    }
    if (pk == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) accw[hh][pc * 8 + e] = acc[hh][e];
    }
  }
};

}  // namespace dsa
