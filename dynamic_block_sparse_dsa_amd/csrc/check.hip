// Selection validator: counts, without trapping, the ways an index array
// breaks the rules the selection calls write it by -- the kept count of a
// row against the selection rule, ids outside the row's visible range, pairs
// that are not strictly ascending (which covers repeats), forced blocks that
// are missing, and padding past the count that is not -1.  A debug aid for
// index arrays that come from outside the library: the attention kernels
// only clamp what they read.
//
// The rules restated here (independently of the selection kernels, so that
// a fault in one shows up in the other) are those of the block selection in
// "dynamic sparse attention explainer", section "基于Top-k选择的局部-全局混合"
// (global anchors plus a local window, the best other blocks up to the
// budget), with the threshold and entropy variants of DeepSeek NSA article
// section 2.2 and the explainer's "工程实践建议", and the token selection of
// the DeepSeek-V3.2 lightning indexer (forced first token and diagonal, the
// best others up to topk).
//
// One thread per row; each workgroup sums its rows' counts through LDS and
// adds them to the report with one 64-bit atomic per slot.  The report is
// cleared by a one-workgroup kernel launched first on the same stream (no
// memset node, so the pair can be graph-captured).
#include "dsa_internal.hpp"

namespace dsa {

namespace {

// forced ids of a row that sees `visible` ids: [0, na) and [ws, visible)
struct Forced {
  int na, ws;
  __device__ int count(int visible) const { return na + (visible - ws); }
  __device__ bool has(int j) const { return j < na || j >= ws; }
};

__device__ Forced forced_of(const CheckArgs& a, int visible) {
  Forced f;
  f.na = min(a.anchors, visible);
  f.ws = max(visible - a.window, f.na);
  return f;
}

// [lo, hi] for the kept count of a row that sees `visible` ids
__device__ void count_range(const CheckArgs& a, int visible, int nf, int& lo, int& hi) {
  int64_t k;
  if (a.sel_mode == DSA_SELECT_THRESHOLD) {
    lo = nf;
    hi = (int)min<int64_t>((int64_t)nf + a.cand_cap, visible);
    return;
  }
  if (a.sel_mode == DSA_SELECT_ENTROPY) {
    lo = min(max(a.k_min, nf), visible);
    hi = min(max(a.k_max, nf), visible);
    return;
  }
  k = a.topk > 0 ? a.topk : ((int64_t)a.topk_num * visible + a.topk_den - 1) / a.topk_den;
  k = min<int64_t>(max<int64_t>(k, nf), visible);
  lo = hi = (int)k;
}

__global__ __launch_bounds__(64) void check_clear_kernel(unsigned long long* report) {
  if (threadIdx.x < DSA_CHECK_N) report[threadIdx.x] = 0ull;
}

__global__ __launch_bounds__(256) void check_kernel(CheckArgs a) {
  __shared__ unsigned long long part[DSA_CHECK_N];
  if (threadIdx.x < DSA_CHECK_N) part[threadIdx.x] = 0ull;
  __syncthreads();
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r < a.n_rows) {
    int visible;
    if (a.layout == DSA_LAYOUT_PREFILL) visible = (int)(r % a.period) + 1;
    else if (a.layout == DSA_LAYOUT_DECODE) visible = a.period;
    else {
      const int len = min(max(a.lengths[r / a.per_seq], 0), a.capacity);
      visible = (len + a.block - 1) / a.block;
    }
    const int32_t* row = a.idx + r * a.kmax;
    int n;
    if (a.cnt) n = a.cnt[r];
    else {  // the count is the length of the list before the -1 padding
      n = 0;
      while (n < a.kmax && row[n] != -1) ++n;
    }
    const Forced f = forced_of(a, visible);
    const int nf = f.count(visible);
    int lo, hi;
    count_range(a, visible, nf, lo, hi);
    const unsigned long long bad_count = (n < lo || n > hi || n > a.kmax) ? 1ull : 0ull;
    n = min(max(n, 0), a.kmax);
    unsigned long long bad_range = 0, bad_order = 0, bad_pad = 0;
    int hits = 0, prev = -1;
    for (int t = 0; t < n; ++t) {
      const int e = row[t];
      bad_range += (e < 0 || e >= visible) ? 1ull : 0ull;
      bad_order += (t > 0 && e <= prev) ? 1ull : 0ull;
      hits += (e >= 0 && e < visible && f.has(e)) ? 1 : 0;
      prev = e;
    }
    for (int t = n; t < a.kmax; ++t) bad_pad += row[t] != -1 ? 1ull : 0ull;
    atomicAdd(&part[DSA_CHECK_ROWS], 1ull);
    if (bad_count) atomicAdd(&part[DSA_CHECK_COUNT], 1ull);
    if (bad_range) atomicAdd(&part[DSA_CHECK_RANGE], bad_range);
    if (bad_order) atomicAdd(&part[DSA_CHECK_ORDER], bad_order);
    if (hits < nf) atomicAdd(&part[DSA_CHECK_FORCED], (unsigned long long)(nf - hits));
    if (bad_pad) atomicAdd(&part[DSA_CHECK_PADDING], bad_pad);
  }
  __syncthreads();
  if (threadIdx.x < DSA_CHECK_N && part[threadIdx.x]) atomicAdd(&a.report[threadIdx.x], part[threadIdx.x]);
}

}  // namespace

hipError_t launch_check(const CheckArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(64), 0, stream, a.report);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_rows == 0) return e;
  hipLaunchKernelGGL(check_kernel, dim3((uint32_t)((a.n_rows + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dsa
