// Host-side planning shared by the C ABI and the launchers: how a decode step
// splits its keys, and how the fused token selection cuts rows into key
// chunks.  Plain C++ with no device code, so the C ABI layer and this file
// can also be built for the host alone (the sanitizer test does).
#include <algorithm>

#include "dsa_internal.hpp"

namespace dsa {

int decode_splits(int S, int Hkv, int kmax) {
  const int64_t units = (int64_t)S * Hkv;
  if (units == 0 || kmax == 0) return 1;
  int64_t want = (DEC_TARGET_WG + units - 1) / units;
  if (want < 1) want = 1;
  if (want > kmax) want = kmax;
  if (want > DEC_MAX_SPLITS) want = DEC_MAX_SPLITS;
  const int bps = (int)((kmax + want - 1) / want);
  return (kmax + bps - 1) / bps;  // every split gets at least one block
}

IndexTopkPlan plan_index_topk(int B, int N, int kmax) {
  IndexTopkPlan pl{};
  const int n_kt = (N + 63) / 64;
  // chunks of at least 32 key tiles: at N = 4096 two chunks of 32 (384 units)
  // take 105 instead of 130 us; shorter or more chunks cost more than they
  // balance at N >= 8192 (per-unit cuts and a longer merge)
  pl.kct = std::max(32, (n_kt + INDEX_TOPK_MAX_CHUNKS - 1) / INDEX_TOPK_MAX_CHUNKS);
  pl.nch = std::max(1, (n_kt + pl.kct - 1) / pl.kct);
  pl.mw = std::max(kmax, 1);
  pl.ws_bytes = pl.nch > 1 ? (size_t)B * N * pl.nch * (8 * (size_t)pl.mw + 4) : 0;
  return pl;
}

}  // namespace dsa
