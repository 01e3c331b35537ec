// Drives every entry point of the C ABI through its argument checks, size
// queries and launch dispatch, with the kernel launchers replaced by host
// stubs (stub_launchers.cpp), under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Prints "abi driver ok" and exits 0 when every
// call returned the expected status; any sanitizer report aborts the run.
#include <cstdio>
#include <cstring>

#include "dsa.h"

extern "C" long long stub_launches;

static int fails = 0;
#define EXPECT(expr, want)                                                                                  \
  do {                                                                                                      \
    const long long rc_ = (long long)(expr);                                                                \
    if (rc_ != (long long)(want)) {                                                                         \
      std::printf("FAIL line %d: %s -> %lld, expected %lld (%s)\n", __LINE__, #expr, rc_, (long long)(want), \
                  dsa_last_error());                                                                        \
      ++fails;                                                                                              \
    }                                                                                                       \
  } while (0)

static dsa_shape mk(int B, int Hq, int Hkv, int N, int d, int b, int topk, int num = 0, int den = 1,
                    unsigned flags = 3) {
  dsa_shape s;
  std::memset(&s, 0, sizeof(s));
  s.batch = B, s.n_q_heads = Hq, s.n_kv_heads = Hkv, s.seq_len = N, s.head_dim = d, s.block = b;
  s.topk = topk, s.topk_num = num, s.topk_den = den, s.flags = flags;
  return s;
}

static dsa_index_shape mki(int B, int Hq, int Hkv, int N, int d, int dI, int topk, unsigned flags = 3) {
  dsa_index_shape s;
  std::memset(&s, 0, sizeof(s));
  s.batch = B, s.n_q_heads = Hq, s.n_kv_heads = Hkv, s.seq_len = N, s.head_dim = d;
  s.n_index_heads = DSA_INDEX_HEADS, s.index_dim = dI, s.topk = topk, s.flags = flags;
  return s;
}

int main() {
  char fake[256];  // a stand-in device address: the stub launchers never dereference it
  void* P = fake;
  float* F = reinterpret_cast<float*>(fake);
  int32_t* I = reinterpret_cast<int32_t*>(fake);
  uint8_t* U = reinterpret_cast<uint8_t*>(fake);
  uint32_t* W = reinterpret_cast<uint32_t*>(fake);
  int64_t* L = reinterpret_cast<int64_t*>(fake);
  const size_t BIG = (size_t)1 << 60;  // workspace sizes are only compared, never touched
  int32_t km = 0;

  for (int st = 1; st >= -6; --st) EXPECT(dsa_status_str(st) != nullptr, 1);

  // ---- prefill and decode shapes of every size class, including the largest workloads
  const dsa_shape good[] = {
      mk(1, 2, 2, 1024, 64, 64, 4),        mk(1, 32, 32, 8192, 128, 64, 16), mk(1, 32, 8, 32768, 128, 64, 0, 15, 100),
      mk(1, 16, 16, 131072, 128, 128, 64), mk(3, 6, 2, 1000, 64, 128, 3),    mk(2, 8, 1, 777, 128, 64, 1, 0, 1, 0),
      mk(1, 4, 4, 1, 64, 64, 4),           mk(5, 8, 2, 64 * 4096, 128, 64, 4096),
  };
  for (const dsa_shape& s : good) {
    EXPECT(dsa_kmax(&s) >= 0, 1);
    EXPECT(dsa_prefill_kmax(&s, &km), DSA_OK);
    const long long before = stub_launches;
    EXPECT(dsa_block_means(&s, s.n_q_heads, P, F, nullptr), DSA_OK);
    EXPECT(dsa_block_scores(&s, P, P, F, nullptr), DSA_OK);
    EXPECT(dsa_block_scores_from_means(&s, F, F, F, nullptr), DSA_OK);
    EXPECT(dsa_select_topk(&s, F, I, I, nullptr), DSA_OK);
    EXPECT(dsa_sparse_attn_fwd(&s, P, P, P, I, I, P, F, nullptr), DSA_OK);
    EXPECT(dsa_prefill(&s, P, P, P, P, F, I, I, P, BIG, nullptr), DSA_OK);
    EXPECT(dsa_prefill(&s, P, P, P, P, nullptr, I, I, P, BIG, nullptr), DSA_OK);
    const size_t pw = dsa_prefill_workspace_bytes(&s);
    if (pw > 0) EXPECT(dsa_prefill(&s, P, P, P, P, F, I, I, P, pw - 1, nullptr), DSA_ERR_WORKSPACE);
    EXPECT(dsa_sparse_attn_bwd(&s, P, P, P, P, F, P, I, I, P, P, P, P, BIG, nullptr), DSA_OK);
    const size_t bw = dsa_attn_bwd_workspace_bytes(&s);
    if (bw > 0) EXPECT(dsa_sparse_attn_bwd(&s, P, P, P, P, F, P, I, I, P, P, P, P, bw - 1, nullptr), DSA_ERR_WORKSPACE);
    EXPECT(stub_launches > before, 1);
    // decode of the same sizes (group sizes 1, 2, 4, 8 only)
    const int G = s.n_q_heads / s.n_kv_heads;
    if (G == 1 || G == 2 || G == 4 || G == 8) {
      EXPECT(dsa_decode_kmax(&s, &km), DSA_OK);
      EXPECT(dsa_kv_block_means(&s, P, F, nullptr), DSA_OK);
      const size_t dw = dsa_decode_workspace_bytes(&s);
      EXPECT(dsa_decode(&s, P, P, P, F, P, F, I, P, BIG, nullptr), DSA_OK);
      EXPECT(dsa_decode(&s, P, P, P, F, P, nullptr, I, P, BIG, nullptr), DSA_OK);
      if (dw > 0) EXPECT(dsa_decode(&s, P, P, P, F, P, F, I, P, dw - 1, nullptr), DSA_ERR_WORKSPACE);
      const int rc = dsa_decode_noalloc(&s, P, P, P, F, P, F, I, nullptr);
      EXPECT(rc == DSA_OK || (rc == DSA_ERR_UNSUPPORTED && dw > DSA_DECODE_NOALLOC_MAX_BYTES), 1);
      const int mb = (s.seq_len + s.block - 1) / s.block;
      EXPECT(dsa_paged_decode(&s, P, P, P, F, 1000, I, mb, I, P, F, I, I, nullptr), DSA_OK);
      EXPECT(dsa_paged_kv_append(&s, P, P, I, mb, I, P, P, F, 1000, nullptr), DSA_OK);
      EXPECT(dsa_paged_kv_block_means(&s, P, I, mb, I, F, 1000, nullptr), DSA_OK);
      EXPECT(dsa_paged_quantize_fp8(&s, P, P, 1000, U, U, F, F, nullptr), DSA_OK);
      EXPECT(dsa_paged_decode_fp8(&s, P, U, U, F, F, F, 1000, I, mb, I, P, F, I, I, nullptr), DSA_OK);
      EXPECT(dsa_paged_kv_append_fp8(&s, P, P, I, mb, I, U, U, F, F, F, 1000, nullptr), DSA_OK);
      EXPECT(dsa_paged_kv_block_means_fp8(&s, U, F, I, mb, I, F, 1000, nullptr), DSA_OK);
      EXPECT(dsa_check_block_selection(&s, DSA_LAYOUT_DECODE, I, nullptr, nullptr, L, nullptr), DSA_OK);
      EXPECT(dsa_check_block_selection(&s, DSA_LAYOUT_PAGED, I, I, I, L, nullptr), DSA_OK);
      EXPECT(dsa_check_block_selection(&s, DSA_LAYOUT_PAGED, I, I, nullptr, L, nullptr), DSA_ERR_NULL);
    }
    EXPECT(dsa_check_block_selection(&s, DSA_LAYOUT_PREFILL, I, I, nullptr, L, nullptr), DSA_OK);
    EXPECT(dsa_check_block_selection(&s, DSA_LAYOUT_PREFILL, I, nullptr, nullptr, L, nullptr), DSA_ERR_NULL);
    EXPECT(dsa_check_block_selection(&s, DSA_LAYOUT_PREFILL, I, I, nullptr, nullptr, nullptr), DSA_ERR_NULL);
    EXPECT(dsa_check_block_selection(&s, 3, I, I, I, L, nullptr), DSA_ERR_SHAPE);
  }
  EXPECT(dsa_indices_to_bitmap(I, I, 4096, 16, 128, W, nullptr), DSA_OK);
  EXPECT(dsa_indices_to_bitmap(I, nullptr, 4096, 16, 128, W, nullptr), DSA_OK);

  // ---- errors: every validation path returns before anything is launched
  const long long launched = stub_launches;
  const dsa_shape ok = mk(1, 4, 2, 1024, 128, 64, 4);
  EXPECT(dsa_kmax(nullptr), DSA_ERR_NULL);
  EXPECT(dsa_prefill_kmax(&ok, nullptr), DSA_ERR_NULL);
  EXPECT(dsa_sparse_attn_fwd(&ok, nullptr, P, P, I, I, P, F, nullptr), DSA_ERR_NULL);
  EXPECT(dsa_prefill(&ok, P, P, P, P, F, I, I, nullptr, BIG, nullptr), DSA_ERR_WORKSPACE);
  EXPECT(dsa_select_topk(&ok, F, nullptr, I, nullptr), DSA_ERR_NULL);
  const dsa_shape bad[] = {
      mk(-1, 4, 2, 1024, 128, 64, 4),           mk(1, 0, 2, 1024, 128, 64, 4),  mk(1, 5, 2, 1024, 128, 64, 4),
      mk(1, 4, 2, 1024, 96, 64, 4),             mk(1, 4, 2, 1024, 128, 32, 4),  mk(1, 4, 2, 1024, 128, 64, -1),
      mk(1, 4, 2, 1024, 128, 64, 4, 0, 1, 8),   mk(1, 4, 2, 1024, 128, 64, 0, 0, 1, 0), mk(1, 4, 2, 1024, 128, 64, 0, 1, 0),
      mk(1, 4, 2, 1024, 128, 64, 0, -1, 4),     mk(1, 4, 2, 64 * 4097, 128, 64, 4),
      mk(1 << 20, 1 << 10, 1 << 10, 1 << 20, 128, 64, 4),
  };
  for (const dsa_shape& s : bad) {
    EXPECT(dsa_prefill_kmax(&s, &km) < 0, 1);
    EXPECT(dsa_prefill(&s, P, P, P, P, F, I, I, P, BIG, nullptr) < 0, 1);
    EXPECT(dsa_decode(&s, P, P, P, F, P, F, I, P, BIG, nullptr) < 0, 1);
    EXPECT(dsa_prefill_workspace_bytes(&s), 0);
  }
  dsa_shape thr = ok;
  thr.select_mode = DSA_SELECT_THRESHOLD, thr.threshold = 1.5f;
  EXPECT(dsa_prefill_kmax(&thr, &km), DSA_ERR_SHAPE);
  dsa_shape ent = ok;
  ent.select_mode = DSA_SELECT_ENTROPY, ent.k_min = 5, ent.k_max = 2;
  EXPECT(dsa_prefill_kmax(&ent, &km), DSA_ERR_SHAPE);
  const dsa_shape g12 = mk(2, 24, 2, 4096, 128, 64, 8);  // decode group of 12: not built
  EXPECT(dsa_decode_kmax(&g12, &km), DSA_ERR_UNSUPPORTED);
  EXPECT(stub_launches, launched);

  // ---- token indexer
  const dsa_index_shape igood[] = {mki(1, 32, 8, 8192, 128, 128, 64), mki(1, 32, 8, 32768, 128, 128, 64),
                                   mki(2, 4, 2, 4200, 64, 64, 128), mki(1, 2, 1, 1, 64, 64, 4),
                                   mki(1, 8, 1, 3000, 128, 128, 129)};
  for (const dsa_index_shape& s : igood) {
    EXPECT(dsa_index_kmax(&s, &km), DSA_OK);
    const size_t iw = dsa_index_workspace_bytes(&s);
    const bool fused = km <= DSA_INDEX_TOPK_MAX_KEEP;
    EXPECT(dsa_index_topk(&s, P, P, F, I, I, P, BIG, nullptr), fused ? DSA_OK : DSA_ERR_UNSUPPORTED);
    if (fused && iw > 0) EXPECT(dsa_index_topk(&s, P, P, F, I, I, P, iw - 1, nullptr), DSA_ERR_WORKSPACE);
    EXPECT(dsa_token_attn_fwd(&s, P, P, P, I, I, P, F, nullptr), DSA_OK);
    const int rc = dsa_index_prefill(&s, P, P, F, P, P, P, P, F, I, I, P, BIG, nullptr);
    EXPECT(rc == DSA_OK || (!fused && s.seq_len > DSA_MAX_TOKENS), 1);
    EXPECT(dsa_check_token_selection(&s, I, I, L, nullptr), DSA_OK);
    EXPECT(dsa_check_token_selection(&s, I, nullptr, L, nullptr), DSA_OK);
    EXPECT(dsa_check_token_selection(&s, I, I, nullptr, nullptr), DSA_ERR_NULL);
    if (s.seq_len <= DSA_MAX_TOKENS) {
      EXPECT(dsa_index_scores(&s, P, P, F, F, nullptr), DSA_OK);
      EXPECT(dsa_select_tokens(&s, F, I, I, nullptr), DSA_OK);
    }
  }
  const dsa_index_shape ibad[] = {mki(1, 32, 8, 8192, 96, 128, 64), mki(1, 32, 8, 8192, 128, 100, 64),
                                  mki(1, 32, 8, 8192, 128, 128, 0), mki(1, 6, 4, 8192, 128, 128, 64),
                                  mki(1, 32, 8, 8192, 128, 128, 64, 4)};
  for (const dsa_index_shape& s : ibad) EXPECT(dsa_index_kmax(&s, &km) < 0, 1);

  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("abi driver ok (%lld launches stubbed)\n", stub_launches);
  return 0;
}
