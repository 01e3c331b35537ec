// Pieces of the decode attention shared by the contiguous-cache kernels
// (decode.hip) and the paged-cache kernel (decode_paged.hip): DPP group sums
// and one wave's online-softmax attention over 32-key chunks (WaveAttn).
#pragma once

#include "attn_common.hpp"

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
  __device__ __forceinline__ float kscale(int, int) const { return 1.f; }
  __device__ __forceinline__ float vscale(int, int) const { return 1.f; }
  __device__ __forceinline__ u32x4 vrow(int v) const { return vv[v]; }
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
// K scale multiplies the key's logit and the V scale its softmax weight.  A lane's key codes are two 16-byte runs of its
// key row, bytes 64 h + 16 (lane / 16) .. + 15 (h = 0, 1): fragment ks holds
// dims 64 (ks / 2) + 16 (lane / 16) + 8 (ks % 2) .. + 7, a permutation of the
// bf16 layout's dims ks * 32 + 8 (lane / 16) .. + 7 that the query fragments
// follow (WaveAttn::init_rows with k16), so each load moves 16 bytes.
template <int D, int G>
struct ChunkRegs8 {
  using C = DecCfg<D, G>;
  u32x4 kq[C::SUB][D / 64];
  u32x2 vv[C::VPL];
  f32x4 ks[C::SUB], vs[C::SUB];
  __device__ __forceinline__ u32x4 kfrag(int sb, int k) const {
    const u32x4 w = kq[sb][k >> 1];
    return fp8x8_to_bf16x8((k & 1) ? (u32x2){w[2], w[3]} : (u32x2){w[0], w[1]});
  }
  __device__ __forceinline__ u32x4 vrow(int v) const { return fp8x8_to_bf16x8(vv[v]); }
  __device__ __forceinline__ float kscale(int sb, int j) const { return ks[sb][j]; }
  __device__ __forceinline__ float vscale(int sb, int j) const { return vs[sb][j]; }
};

// Row swizzle of a wave's V tile in LDS ([32 keys][D] bf16): the 16-byte
// chunk index is XORed with vsw(row), so that the 32 lanes of two 16-lane
// groups of a transposed read (4 consecutive rows x 4 dims each) hit 64
// distinct four-byte banks.
template <int D>
__device__ __forceinline__ int dec_vsw(int r) {
  return D == 128 ? 2 * ((r & 3) + 4 * ((r >> 2) & 1)) : 2 * (((r >> 1) & 1) + 2 * ((r >> 2) & 1));
}

// One wave's online-softmax state for the G query heads of a unit, and the
// per-chunk work, both products on v_mfma_f32_16x16x32_bf16 with the group's
// heads as the 16 columns.  S = K Q^T (key rows as the A operand) leaves head
// n = lane % 16 in the lane and keys 16 sb + 4 (lane / 16) + j in its slots,
// which is already the B operand order of O^T += V^T P^T.  The V rows go from
// registers into the wave's LDS tile and come back transposed
// (ds_read_b64_tr_b16) as the A operand, in the same key order.  The weights
// enter as two bf16 terms, P = hi + lo (hi the bf16 rounding of P, lo that of
// the remainder), so P V keeps about 16 bits of each weight; accumulation is
// fp32.
template <int D, int G>
struct WaveAttn {
  using C = DecCfg<D, G>;
  static constexpr int NDB = D / 16;  // 16-dim blocks of O
  u32x4 qf[D / 32];
  float m_run, l_run;  // head n's state (lanes with n < G)
  f32x4 acc[NDB];      // head n's dims 16 db + 4 (lane / 16) + j
  int lane, n, lq, pc, pk;

  __device__ __forceinline__ void init(const DecodeArgs& a, int64_t s, int g) { init(a.q, a.Hq, s, g); }

  // q [S, Hq, D]: the group's heads of sequence s
  __device__ __forceinline__ void init(const uint16_t* q, int Hq, int64_t s, int g, bool k16 = false) {
    init_rows(q + (s * Hq + g * G) * (int64_t)D, D, k16);
  }

  // query row of the group's head hh at q0 + hh * head_stride; k16: the
  // fragment dims of ChunkRegs8 (16-byte FP8 key loads)
  __device__ __forceinline__ void init_rows(const uint16_t* q0, int64_t head_stride, bool k16 = false) {
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
      const int d0 = k16 ? 64 * (ks >> 1) + 16 * lq + 8 * (ks & 1) : ks * 32 + 8 * lq;
      if (n < G) qf[ks] = *reinterpret_cast<const u32x4*>(q0 + n * head_stride + d0);
    }
    m_run = -__builtin_inff();
    l_run = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = (f32x4){0, 0, 0, 0};
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

  // the FP8 chunk: codes and the row scales of this lane's keys (ksb, vsb
  // are the tile's BLK scales); scales of keys past L are 0
  __device__ __forceinline__ void load8(ChunkRegs8<D, G>& r, const uint8_t* kb, const uint8_t* vb, const float* ksb,
                                        const float* vsb, int key0, int L) const {
#pragma unroll
    for (int sb = 0; sb < C::SUB; ++sb) {
      const int key = min(key0 + sb * 16 + (lane & 15), L - 1);
#pragma unroll
      for (int h = 0; h < D / 64; ++h)
        r.kq[sb][h] =
            __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (int64_t)key * D + 64 * h + 16 * lq));
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

  // fold the chunk into the state; vt is this wave's LDS tile
  template <class Regs>
  __device__ __forceinline__ void step(const Regs& r, int key0, int L, float scale_log2, LDS_AS uint16_t* vt) {
    const float NEG_INF = -__builtin_inff();
    // V rows into the tile: lane (pk, pc) holds dims 8 pc .. of rows pk + KGR v
#pragma unroll
    for (int v = 0; v < C::VPL; ++v) {
      const int rr = pk + C::KGR * v;
      *reinterpret_cast<LDS_AS u32x4*>(vt + rr * D + (pc ^ dec_vsw<D>(rr)) * 8) = r.vrow(v);
    }
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
    u32x4 ph, pl;  // B operands: the weights' bf16 rounding and that of the rest
#pragma unroll
    for (int sb = 0; sb < C::SUB; ++sb) {
      float w[4];
      __bf16 h[4], l[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float pv = __builtin_amdgcn_exp2f(sc[sb][j] - m_run);
        lsum += pv;
        w[j] = pv * r.vscale(sb, j);  // V scale folded into the weight
        h[j] = (__bf16)w[j];
        l[j] = (__bf16)(w[j] - (float)h[j]);
      }
      ph[2 * sb] = __builtin_bit_cast(uint32_t, (bf16x2_t){h[0], h[1]});
      ph[2 * sb + 1] = __builtin_bit_cast(uint32_t, (bf16x2_t){h[2], h[3]});
      pl[2 * sb] = __builtin_bit_cast(uint32_t, (bf16x2_t){l[0], l[1]});
      pl[2 * sb + 1] = __builtin_bit_cast(uint32_t, (bf16x2_t){l[2], l[3]});
    }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    // the tile writes above come before the transposed reads (one wave's LDS
    // operations complete in order; the fence keeps the compiler's order)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int src = lane & 15;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      u32x4 va;
#pragma unroll
      for (int sg = 0; sg < 2; ++sg) {
        const int rr = 4 * lq + 16 * sg + (src >> 2);  // key row of the chunk
        const int d0 = db * 16 + 4 * (src & 3);        // first of this source lane's 4 dims
        const int ch = (d0 >> 3) ^ dec_vsw<D>(rr);
        const LDS_AS char* addr = reinterpret_cast<const LDS_AS char*>(vt + rr * D + ch * 8) + (d0 & 7) * 2;
        const u32x2 w2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)addr));
        va[2 * sg] = w2[0];
        va[2 * sg + 1] = w2[1];
      }
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(ph), acc[db], 0, 0, 0);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pl), acc[db], 0, 0, 0);
    }
    // the next chunk's tile writes come after these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // leave (max, sum, acc[d]) per head in LDS
  __device__ __forceinline__ void to_lds(float* mw, float* lw, float (*accw)[D]) {
    if (n < G) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) accw[n][db * 16 + 4 * lq + j] = acc[db][j];
      if (lq == 0) {
        mw[n] = m_run;
        lw[n] = l_run;
      }
    }
  }
};

}  // namespace dsa
