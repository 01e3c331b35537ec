// Top-k selection of one row by one wavefront (shared by the prefill select
// kernel and the fused decode select kernel).
//
// Method: "dynamic sparse attention explainer" (zblog.xzdbk.com/559.html),
// "基于Top-k选择的局部-全局混合": keep the k best-scoring blocks plus the
// anchors (the first blocks, the sink) and a local window (the last visible
// blocks, ending at the row's own).  The budget k is fixed or a fraction of
// the visible blocks, or comes from the row's block distribution (softmax of
// its visible block scores): the number of candidates whose share reaches a
// threshold (DeepSeek NSA article, section 2.2), or ceil(exp(entropy))
// ("模型精度与稀疏度的动态平衡" and "工程实践建议" of the explainer).
//
// Lane l owns the contiguous run of R blocks starting at l * R (index order),
// so the final compaction is an exclusive scan.  Each visible non-forced
// block is a candidate whose score becomes an order-preserving uint32 key.
// The m-th largest candidate key T is found by a most-significant-bit-first
// search over the key bits: starting from the common prefix of the largest and
// smallest candidate key, each step tries to set the next bit and keeps it
// when at least m candidates are >= the trial value.  A count is R vector
// compares into wave masks whose bits the scalar unit counts, so the search
// needs no LDS and no barrier, and all its control flow is wave-uniform.
// When a trial value has exactly m candidates at or above it, those are the
// answer and the search stops early; otherwise the candidates above T are
// kept and, among the ones equal to T, the lowest indices fill the rest
// (ties go to the lower block).
//
// Fast path (R >= 16, m <= 64): each lane splits its keys into 4 groups; the
// m-th largest of the 256 group maxima, t0, is a lower bound of T (m distinct
// keys are >= t0).  Only candidates >= t0 can be kept; when there are at most
// 128 of them they are compacted in index order through 1 KiB of LDS, two per
// lane, and the same search runs on those.  The forced blocks are a prefix
// (anchors) and a suffix (window) of the visible range, so they go first and
// last around the candidates.
#pragma once

#include "dsa_internal.hpp"

namespace dsa {

// number of keys >= c over the R keys of each of the 64 lanes (all active):
// one compare per key into a wave mask, counted on the scalar unit, so the
// result is wave-uniform
template <int R>
__device__ __forceinline__ int wave_count_ge(const uint32_t (&key)[R], uint32_t c) {
  int n = 0;
#pragma unroll
  for (int e = 0; e < R; ++e) n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(key[e] >= c));
  return n;
}

// inclusive prefix sum over the 64 lanes (all active): DPP shifts by 1, 2,
// 4, 8 within each row of 16 lanes, then the row totals broadcast forward
// (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3)
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// max / min over the 64 lanes, returned as wave-uniform values: DPP within
// rows of 16 lanes, then the four row results through readlane
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// lanes below this one whose bit is set in mask
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Largest T >= 1 with at least m of the values v[0..C-1] of the 64 lanes
// >= T (0 if fewer than m values are >= 1; a 0 never counts).  *exact is set
// when exactly m values are >= T.  With EARLY the search stops at the first
// trial value with exactly m values at or above it (T then has only its
// leading bits and can lie well below the m-th largest value); without it T
// is the m-th largest value itself.
template <int C, bool EARLY = true>
__device__ __forceinline__ uint32_t wave_kth_largest(const uint32_t (&v)[C], int m, bool* exact) {
  uint32_t T = 0;
  *exact = false;
  for (int b = 31; b >= 0; --b) {
    const uint32_t trial = T | (1u << b);
    int n = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(v[c] >= trial));
    if (n >= m) {
      T = trial;
      if (EARLY && n == m) {
        *exact = true;
        break;
      }
    }
  }
  return T;
}

// Budget of a threshold- or entropy-mode row (wave-uniform), from the
// row's block distribution p_j = exp(s_j - mx) / z over blocks 0 .. nv-1:
// THRESHOLD keeps the candidates (na <= j < ws) with p_j >= tau, i.e.
// s_j >= mx + ln(tau z), at most p.cand_cap of them; ENTROPY keeps
// ceil(exp(H)) blocks, H = ln z - (sum_j e_j (s_j - mx)) / z, clamped to
// [k_min, k_max].  All in fp32.
template <int R, bool LDS_T>
__device__ int64_t dist_budget(const float* srow, int nv, const TopkParams& p, int na, int ws) {
  const int lane = threadIdx.x & 63;
  const int j0 = lane * R;
  float sv[R];
#pragma unroll
  for (int e = 0; e < R; ++e) {
    const int j = j0 + e;
    if constexpr (LDS_T) sv[e] = ((const __attribute__((address_space(3))) float*)srow)[e * 64 + lane];
    else sv[e] = j < nv ? srow[j] : 0.f;
  }
  float mx = -__builtin_inff();
#pragma unroll
  for (int e = 0; e < R; ++e)
    if (j0 + e < nv) mx = fmaxf(mx, sv[e]);
  mx = wave_max_f32(mx);
  float z = 0.f, a = 0.f;
#pragma unroll
  for (int e = 0; e < R; ++e)
    if (j0 + e < nv) {
      const float t = sv[e] - mx;
      const float ex = expf(t);
      z += ex;
      a += ex * t;
    }
  z = wave_sum_f32(z);
  a = wave_sum_f32(a);
  const int nf = na + (nv - ws);
  if (p.mode == DSA_SELECT_THRESHOLD) {
    const float thr = mx + logf(p.threshold * z);
    int c = 0;
#pragma unroll
    for (int e = 0; e < R; ++e) {
      const int j = j0 + e;
      c += __builtin_popcountll(__builtin_amdgcn_ballot_w64(j >= na && j < ws && sv[e] >= thr));
    }
    return nf + min(c, p.cand_cap);
  }
  const float h = logf(z) - a / z;
  const int k = (int)ceilf(expf(h));
  return min(max(k, p.k_min), p.k_max);
}

// Select from the scores of blocks 0 .. nv-1, nv <= 64 * R.  Without LDS_T,
// srow[j] is block j's score (global or LDS); with LDS_T, srow is an LDS
// array of 64 * R scores laid out so that block j = l * R + e sits at
// srow[e * 64 + l] (conflict-free reads), entries past nv are ignored.
// Writes the kept blocks ascending to out[0 ..], pads out[.. kmax-1] with -1
// and returns the number kept.  Called by all 64 lanes of one wave; lds_key
// and lds_idx are 128-entry LDS arrays private to the wave.
template <int R, bool LDS_T = false>
__device__ int wave_select_row(const float* srow, int nv, TopkParams p, int32_t* out, int kmax, uint32_t* lds_key,
                               int32_t* lds_idx) {
  const int lane = threadIdx.x & 63;
  // forced: the prefix [0, na) (anchors) and the suffix [ws, nv) (window)
  const int na = min(p.anchors, nv);
  const int ws = max(nv - p.window, na);
  const int nf = na + (nv - ws);
  int64_t budget;
  if (p.mode == DSA_SELECT_TOPK) budget = p.topk > 0 ? (int64_t)p.topk : ((int64_t)p.num * nv + p.den - 1) / p.den;
  else budget = dist_budget<R, LDS_T>(srow, nv, p, na, ws);
  if (budget < nf) budget = nf;
  if (budget > nv) budget = nv;
  const int m = (int)budget - nf;  // candidates to keep
  const int ncand = nv - nf;
  const int j0 = lane * R;

  // key 0 marks a non-candidate in the counts: every trial value is >= 1
  uint32_t key[R];
  uint32_t candbits[(R + 31) / 32];
  uint32_t kmx = 0, kmn = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < (R + 31) / 32; ++w) candbits[w] = 0;
  float sv[R];
  if constexpr (LDS_T) {
    const __attribute__((address_space(3))) float* st = (const __attribute__((address_space(3))) float*)srow;
#pragma unroll
    for (int e = 0; e < R; ++e) sv[e] = st[e * 64 + lane];
  }
#pragma unroll
  for (int e = 0; e < R; ++e) {
    const int j = j0 + e;
    key[e] = 0;
    if (j >= na && j < ws) {
      key[e] = order_key(LDS_T ? sv[e] : srow[j]);
      candbits[e / 32] |= 1u << (e % 32);
      kmx = max(kmx, key[e]);
      kmn = min(kmn, key[e]);
    }
  }

  const bool all = (m >= ncand), none = (m <= 0);
  if (R >= 16 && !all && !none && m <= 64) {
    constexpr int GS = R / 4;  // keys per group
    uint32_t gmax[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      gmax[g] = 0;
#pragma unroll
      for (int e = g * GS; e < (g + 1) * GS; ++e) gmax[g] = max(gmax[g], key[e]);  // 0 for non-candidates
    }
    bool ex;
    const uint32_t t0 = wave_kth_largest<4>(gmax, m, &ex);
    int mine = 0;  // this lane's candidates >= t0
#pragma unroll
    for (int e = 0; e < R; ++e) mine += ((candbits[e / 32] >> (e % 32)) & 1u) && key[e] >= t0;
    const int incl = wave_incl_scan(mine);
    const int ns = __builtin_amdgcn_readlane(incl, 63);
    if (t0 > 0 && ns <= 128) {
      int q = incl - mine;
#pragma unroll
      for (int e = 0; e < R; ++e)
        if (((candbits[e / 32] >> (e % 32)) & 1u) && key[e] >= t0) {
          lds_key[q] = key[e];
          lds_idx[q] = j0 + e;
          ++q;
        }
      wave_lds_sync();
      // survivor positions lane and 64 + lane, in index order
      const bool ok0 = lane < ns, ok1 = lane + 64 < ns;
      const uint32_t k0 = ok0 ? lds_key[lane] : 0u, k1 = ok1 ? lds_key[64 + lane] : 0u;
      const int i0 = ok0 ? lds_idx[lane] : -1, i1 = ok1 ? lds_idx[64 + lane] : -1;
      wave_lds_sync();
      bool exact;
      const uint32_t kk[2] = {k0, k1};  // all >= t0 >= 1 where valid
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
      return total;
    }
  }

  uint32_t T = 0;
  int take_eq = 0x7fffffff;  // candidates equal to T that are kept, in index order
  if (!all && !none) {
    const uint32_t hi = wave_max_u32(kmx), lo = wave_min_u32(kmn);
    const uint32_t diff = hi ^ lo;
    bool exact = false;
    if (diff == 0) {
      T = lo;  // every candidate has the same key
    } else {
      const int top = 31 - __builtin_clz(diff);
      T = top == 31 ? 0u : hi & ~((2u << top) - 1u);  // common prefix: T <= lo, all candidates >= T
      for (int b = top; b >= 0; --b) {
        const uint32_t trial = T | (1u << b);
        const int n_ge = wave_count_ge<R>(key, trial);
        if (n_ge >= m) {
          T = trial;
          if (n_ge == m) {
            exact = true;
            break;
          }
        }
      }
    }
    if (!exact) {
      // T is the m-th largest candidate key: keep the ones above it, then ties
      take_eq = T == 0xffffffffu ? m : m - wave_count_ge<R>(key, T + 1u);
    }
  }

  // rank of each equal-to-T candidate among the equal ones, in index order
  int my_eq = 0;
  if (!all && !none) {
#pragma unroll
    for (int e = 0; e < R; ++e) my_eq += ((candbits[e / 32] >> (e % 32)) & 1u) && key[e] == T;
  }
  int running_eq = wave_incl_scan(my_eq) - my_eq;

  uint32_t selbits[(R + 31) / 32];
#pragma unroll
  for (int w = 0; w < (R + 31) / 32; ++w) selbits[w] = 0;
#pragma unroll
  for (int e = 0; e < R; ++e) {
    const int j = j0 + e;
    if (j >= nv) continue;
    const bool cand = (candbits[e / 32] >> (e % 32)) & 1u;
    bool s;
    if (!cand) s = true;  // forced
    else if (all) s = true;
    else if (none) s = false;
    else if (key[e] > T) s = true;
    else if (key[e] == T) {
      s = running_eq < take_eq;
      ++running_eq;
    } else s = false;
    selbits[e / 32] |= (uint32_t)s << (e % 32);
  }
  int my_sel = 0;
#pragma unroll
  for (int w = 0; w < (R + 31) / 32; ++w) my_sel += __builtin_popcount(selbits[w]);
  const int incl = wave_incl_scan(my_sel);
  int pos = incl - my_sel;
#pragma unroll
  for (int e = 0; e < R; ++e)
    if ((selbits[e / 32] >> (e % 32)) & 1u) out[pos++] = j0 + e;
  const int total = __builtin_amdgcn_readlane(incl, 63);
  for (int e = total + lane; e < kmax; e += 64) out[e] = -1;
  return total;
}

// ---------------------------------------------------------------- workgroup top-k
// Workgroup barrier that orders LDS only: global loads in flight (a caller's
// prefetch into registers) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS words block_select_topk needs as scratch (up to 16 waves): two 256-bin
// histograms, per-wave maxima, minima and scan totals, broadcast slots.
constexpr int BSEL_SCRATCH_WORDS = 2 * 256 + 3 * 16 + 4;

// Plain top-k selection of one row by all NT threads of a workgroup, with the
// result of wave_select_row<R, true> (same forced prefix and suffix, same
// budget, the top m candidates by (score desc, index asc), kept blocks written
// ascending to out and padded with -1 to kmax; returns the number kept).  For
// DSA_SELECT_TOPK rows only.  srow is the LDS score row in the transposed
// layout (block l R + e at srow[e * 64 + l]); out may be global or LDS and is
// complete after the caller's next barrier.  The m-th largest order key is
// found a digit at a time (at most 8 bits per pass, from the highest bit in
// which the candidate keys differ): an LDS histogram of the digit over the
// keys that match the digits fixed so far, one wave walks it from the top to
// the bin holding the m-th key, and the search ends early when that bin holds
// exactly the keys still needed.  Thread t owns blocks t E .. t E + E - 1, so
// one packed prefix sum in thread order ranks the ties at the threshold and
// places every kept block.  Contains LDS-only barriers: every thread must
// call it, and global loads the caller has in flight stay in flight.
template <int R, int NT>
__device__ __forceinline__ int block_select_topk(const float* srow, int nv, const TopkParams& p, int32_t* out,
                                                 int kmax, uint32_t* scratch) {
  constexpr int NW = NT / 64;
  constexpr int E = 64 * R / NT;  // blocks per thread
  static_assert(E >= 1 && E * NT == 64 * R && NW <= 16, "row split");
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint32_t* hist = scratch;             // [2][256]
  uint32_t* wmx = scratch + 512;        // [NW] per-wave maxima of the candidate keys
  uint32_t* wmn = scratch + 512 + 16;   // [NW] minima
  uint32_t* wsc = scratch + 512 + 32;   // [NW] packed scan totals
  uint32_t* bc = scratch + 512 + 48;    // broadcast: digit, need, exact
  const int na = min(p.anchors, nv);
  const int ws = max(nv - p.window, na);
  const int nf = na + (nv - ws);
  int64_t budget = p.topk > 0 ? (int64_t)p.topk : ((int64_t)p.num * nv + p.den - 1) / p.den;
  if (budget < nf) budget = nf;
  if (budget > nv) budget = nv;
  const int m = (int)budget - nf;
  const int ncand = nv - nf;
  const int j0 = t * E;

  if (m <= 0 || m >= ncand) {  // forced blocks only, or every visible block
    const int total = m <= 0 ? nf : nv;
    for (int e = t; e < total; e += NT) out[e] = (m <= 0 && e >= na) ? ws + (e - na) : e;
    for (int e = total + t; e < kmax; e += NT) out[e] = -1;
    return total;
  }

  const __attribute__((address_space(3))) float* st = (const __attribute__((address_space(3))) float*)srow;
  uint32_t key[E];
  bool cand[E];
  uint32_t kmx = 0, kmn = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = j0 + e;
    cand[e] = j >= na && j < ws;
    key[e] = cand[e] ? order_key(st[(j % R) * 64 + j / R]) : 0u;
    if (cand[e]) {
      kmx = max(kmx, key[e]);
      kmn = min(kmn, key[e]);
    }
  }
  kmx = wave_max_u32(kmx);
  kmn = wave_min_u32(kmn);
  if (lane == 0) {
    wmx[wave] = kmx;
    wmn[wave] = kmn;
  }
  hist[t % 512] = 0u;
  if (NT < 512)
    for (int e = t + NT; e < 512; e += NT) hist[e] = 0u;
  lds_barrier();
  uint32_t hi = 0, lo = 0xffffffffu;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    hi = max(hi, wmx[w]);
    lo = min(lo, wmn[w]);
  }

  // digits fixed so far: the keys with (key & M) == P hold the m-th largest,
  // and `need` of them are kept
  uint32_t P = hi, M = 0xffffffffu;
  int need = m;
  if (hi != lo) {
    int top = 31 - __builtin_clz(hi ^ lo);  // highest bit in which candidate keys differ
    M = top == 31 ? 0u : ~((2u << top) - 1u);
    P = hi & M;
    for (int pass = 0;; ++pass) {
      const int shift = max(top - 7, 0);
      const uint32_t dm = (2u << (top - shift)) - 1u;  // digit mask, at most 8 bits
      uint32_t* h = hist + 256 * (pass & 1);
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (cand[e] && (key[e] & M) == P) atomicAdd(&h[(key[e] >> shift) & dm], 1u);
      lds_barrier();
      if (wave == 0) {
        // lane l holds digits dm - 4 l - i (i = 0..3): descending over the lanes
        uint32_t c[4];
        int tot = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d = (int)dm - 4 * lane - i;
          c[i] = d >= 0 ? h[d] : 0u;
          tot += (int)c[i];
        }
        int run = wave_incl_scan(tot) - tot;  // keys in higher digits than this lane's
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (run < need && need <= run + (int)c[i]) {
            bc[0] = (uint32_t)((int)dm - 4 * lane - i);
            bc[1] = (uint32_t)(need - run);
            bc[2] = (uint32_t)(need - run) == c[i];
          }
          run += (int)c[i];
        }
      }
      lds_barrier();
      const uint32_t d = bc[0];
      need = (int)bc[1];
      const bool exact = bc[2] != 0u;
      if (t < 256) h[t] = 0u;  // free for the pass after next (a barrier lies between)
      P |= d << shift;
      M |= dm << shift;
      if (exact || shift == 0) break;
      top = shift - 1;
    }
  }

  // kept: forced, (key & M) > P, or (key & M) == P among the first `need` in
  // index order.  Packed counts (above << 16 | at) in thread order.
  uint32_t v = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = j0 + e;
    const bool forced = j < nv && !cand[e];
    if (forced || (cand[e] && (key[e] & M) > P)) v += 1u << 16;
    else if (cand[e] && (key[e] & M) == P) v += 1u;
  }
  const uint32_t incl = (uint32_t)wave_incl_scan((int)v);
  if (lane == 63) wsc[wave] = incl;
  lds_barrier();
  uint32_t before = incl - v;
  for (int w = 0; w < wave; ++w) before += wsc[w];
  int above = (int)(before >> 16), at = (int)(before & 0xffffu);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = j0 + e;
    const bool forced = j < nv && !cand[e];
    if (forced || (cand[e] && (key[e] & M) > P)) {
      out[above + min(at, need)] = j;
      ++above;
    } else if (cand[e] && (key[e] & M) == P) {
      if (at < need) out[above + at] = j;
      ++at;
    }
  }
  const int total = nf + m;
  for (int e = total + t; e < kmax; e += NT) out[e] = -1;
  return total;
}

// Best m of the keys v[0..C-1] of each lane (0 = not a candidate; lane-major
// runs, so position order is lane * C + c): sets keep[c] and returns the
// number kept, exactly min(m, candidates).  With more than m candidates,
// *lower (if given) receives a value that at least m keys reach.  The m-th largest key T comes from
// an MSB-first search that starts at the common leading bits of the largest
// and smallest candidate key and stops as soon as exactly m keys are >= the
// trial value; otherwise T is the m-th largest key and the keys equal to it
// are kept in position order until m are kept.  All lanes active.
template <int C>
__device__ __forceinline__ int wave_keep_best(const uint32_t (&v)[C], int m, bool (&keep)[C], uint32_t* lower = nullptr) {
  int n = 0;
  uint32_t mx = 0u, mn = ~0u;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(v[c] != 0u));
    if (v[c]) {
      mx = max(mx, v[c]);
      mn = min(mn, v[c]);
    }
  }
  uint32_t T = 1u;
  bool cut = false;
  int take_eq = 0;
  if (n > m) {
    mx = wave_max_u32(mx);
    mn = wave_min_u32(mn);
    const uint32_t x = mx ^ mn;
    int bit = x ? 31 - __builtin_clz(x) : -1;
    T = x ? (mx & ~(uint32_t)(((uint64_t)2 << bit) - 1u)) : mx;
    int nT = n;
    // two bits per step: the three trial values are counted independently
    for (; bit >= 1 && nT > m; bit -= 2) {
      const uint32_t t1 = T | (1u << (bit - 1)), t2 = T | (2u << (bit - 1)), t3 = T | (3u << (bit - 1));
      const int c1 = wave_count_ge<C>(v, t1), c2 = wave_count_ge<C>(v, t2), c3 = wave_count_ge<C>(v, t3);
      if (c3 >= m) {
        T = t3;
        nT = c3;
      } else if (c2 >= m) {
        T = t2;
        nT = c2;
      } else if (c1 >= m) {
        T = t1;
        nT = c1;
      }
    }
    if (bit == 0 && nT > m) {
      const int c = wave_count_ge<C>(v, T | 1u);
      if (c >= m) {
        T |= 1u;
        nT = c;
      }
    }
    cut = nT > m;
    if (cut) take_eq = m - (T == ~0u ? 0 : wave_count_ge<C>(v, T + 1u));
    if (lower) *lower = T;  // at least m of the keys are >= T
  }
  int my_eq = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) my_eq += v[c] == T;
  int r = cut ? wave_incl_scan(my_eq) - my_eq : 0;
  int kept = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    keep[c] = v[c] > T || (v[c] == T && (!cut || r < take_eq));
    r += v[c] == T;
    kept += keep[c];
  }
  return min(n, m);
}

// LDS words the two-round selection needs: a list of up to 64 (key, block)
// per wave, a count and a lower bound per wave (up to 16 waves)
constexpr int BSEL2_SCRATCH_WORDS = 16 * 64 * 2 + 32;

// Budget split of a DSA_SELECT_TOPK row that sees nv blocks: forced prefix
// [0, na), forced suffix [ws, nv), m candidates kept (wave-uniform)
struct TopkRow {
  int na, ws, nf, m;
  __device__ __forceinline__ TopkRow(int nv, const TopkParams& p) {
    na = min(p.anchors, nv);
    ws = max(nv - p.window, na);
    nf = na + (nv - ws);
    int64_t budget = p.topk > 0 ? (int64_t)p.topk : ((int64_t)p.num * nv + p.den - 1) / p.den;
    if (budget < nf) budget = nf;
    if (budget > nv) budget = nv;
    m = (int)budget - nf;
  }
  // rows the two rounds take: some candidates kept, not all, at most 64
  __device__ __forceinline__ bool two_round(int nv) const { return m > 0 && m < nv - nf && m <= 64; }
};

// Round 1 of the two-round selection, run by one wave on its own range of
// blocks w B .. w B + B - 1 (B = 64 R / NW, R / NW consecutive blocks per
// lane): the wave keeps its best m candidates (wave_keep_best) and writes them
// in index order as an LDS list of LS slots (LS >= m) with its count.  srow:
// the LDS score row in the transposed layout (block l R + e at srow[e * 64 +
// l]), already written by this wave for its range (the caller syncs).
template <int R, int NW>
__device__ __forceinline__ void topk_round1(const float* srow, const TopkRow& tr, int ls, uint32_t* scratch2) {
  constexpr int C = R / NW;
  static_assert(C >= 1 && C * NW == R && NW <= 16, "row split");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __attribute__((address_space(3))) float* st = (const __attribute__((address_space(3))) float*)srow;
  uint32_t* lkey = scratch2;                // [NW][ls]
  uint32_t* lblk = scratch2 + 16 * 64;      // [NW][ls]
  uint32_t* lcnt = scratch2 + 2 * 16 * 64;  // [NW]
  uint32_t* lbnd = lcnt + 16;               // [NW]
  uint32_t v[C];
  const int j0 = wave * 64 * C + lane * C;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int j = j0 + c;
    v[c] = (j >= tr.na && j < tr.ws) ? order_key(st[(j % R) * 64 + j / R]) : 0u;
  }
  bool keep[C];
  uint32_t bound = 0u;
  const int kw = wave_keep_best<C>(v, tr.m, keep, &bound);
  int mine = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) mine += keep[c];
  int pos = wave_incl_scan(mine) - mine;
#pragma unroll
  for (int c = 0; c < C; ++c)
    if (keep[c]) {
      lkey[wave * ls + pos] = v[c];
      lblk[wave * ls + pos] = (uint32_t)(j0 + c);
      ++pos;
    }
  if (lane == 0) {
    lcnt[wave] = (uint32_t)kw;
    lbnd[wave] = bound;
  }
}

// Round 2, one wave, after a barrier behind every wave's round 1: the best m
// of the concatenated lists (in index order, so ties again go to the lower
// block), written to out with the forced blocks: anchors, kept ascending,
// window, -1 padding to kmax.  C2 = NW * ls / 64 list slots per lane.
template <int NW, int C2>
__device__ __forceinline__ void topk_round2(const TopkRow& tr, int nv, int32_t* out, int kmax, int ls,
                                            const uint32_t* scratch2) {
  static_assert(C2 * 64 <= 16 * 64, "list slots");
  const int lane = threadIdx.x & 63;
  const uint32_t* lkey = scratch2;
  const uint32_t* lblk = scratch2 + 16 * 64;
  const uint32_t* lcnt = scratch2 + 2 * 16 * 64;
  const uint32_t* lbnd = lcnt + 16;
  // a wave with more than m candidates has m keys >= its bound, so keys below
  // the largest bound cannot be among the best m: dropping them shortens the
  // threshold search
  uint32_t lb = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) lb = max(lb, lbnd[w]);
  uint32_t u[C2], blk[C2];
#pragma unroll
  for (int c = 0; c < C2; ++c) {
    const int q = lane * C2 + c, w = q / ls, i = q - w * ls;
    const bool ok = w < NW && i < (int)lcnt[min(w, NW - 1)];
    const uint32_t k = ok ? lkey[q] : 0u;
    u[c] = k >= lb ? k : 0u;
    blk[c] = ok ? lblk[q] : 0u;
  }
  bool k2[C2];
  wave_keep_best<C2>(u, tr.m, k2);
  int mine = 0;
#pragma unroll
  for (int c = 0; c < C2; ++c) mine += k2[c];
  int o = tr.na + wave_incl_scan(mine) - mine;
#pragma unroll
  for (int c = 0; c < C2; ++c)
    if (k2[c]) out[o++] = (int32_t)blk[c];
  for (int e = lane; e < tr.na; e += 64) out[e] = e;
  for (int e = lane; e < nv - tr.ws; e += 64) out[tr.na + tr.m + e] = tr.ws + e;
  for (int e = tr.nf + tr.m + lane; e < kmax; e += 64) out[e] = -1;
}

// block_select_topk's result for rows that keep at most 64 candidates (and
// see at most 64 R blocks), in two wave-level rounds instead of a workgroup
// radix search (topk_round1 on every wave, a barrier, topk_round2 on wave 0).
// Every thread must call it; out is complete after the caller's next barrier.
template <int R, int NT>
__device__ __forceinline__ int block_select_topk_waves(const float* srow, int nv, const TopkParams& p, int32_t* out,
                                                       int kmax, uint32_t* scratch, uint32_t* scratch2) {
  constexpr int NW = NT / 64;
  const TopkRow tr(nv, p);
  if (!tr.two_round(nv)) return block_select_topk<R, NT>(srow, nv, p, out, kmax, scratch);
  const int ls = tr.m <= 32 ? 32 : 64;
  topk_round1<R, NW>(srow, tr, ls, scratch2);
  lds_barrier();
  if ((threadIdx.x >> 6) == 0) {
    if (ls == 32) topk_round2<NW, NW / 2>(tr, nv, out, kmax, ls, scratch2);
    else topk_round2<NW, NW>(tr, nv, out, kmax, ls, scratch2);
  }
  return tr.nf + tr.m;
}

}  // namespace dsa
