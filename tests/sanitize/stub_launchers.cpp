// Host-only stand-ins for the kernel launchers of libdsa, for the sanitizer
// build of the C ABI layer (api.cpp + plan.cpp): each records that it was
// called and returns success without touching the (fake) device pointers, so
// every argument check, size computation and dispatch decision of the C ABI
// runs on the CPU under AddressSanitizer and UndefinedBehaviorSanitizer.
#include "dsa_internal.hpp"

extern "C" long long stub_launches = 0;

namespace dsa {
static hipError_t hit() {
  ++stub_launches;
  return hipSuccess;
}
hipError_t launch_block_means(const uint16_t*, float*, int64_t, int, int, int, hipStream_t) { return hit(); }
hipError_t launch_block_means2(const uint16_t*, float*, int64_t, const uint16_t*, float*, int64_t, int, int, int,
                               hipStream_t) { return hit(); }
hipError_t launch_block_scores(const float*, const float*, float*, int, int, int, int, int, float, hipStream_t) {
  return hit();
}
hipError_t launch_pooled_scores(const uint16_t*, const uint16_t*, float*, int, int, int, int, int, int, float,
                                hipStream_t) { return hit(); }
hipError_t launch_select_topk(const float*, int32_t*, int32_t*, int64_t, int, int, bool, TopkParams, int, hipStream_t) {
  return hit();
}
hipError_t launch_bitmap(const int32_t*, const int32_t*, uint32_t*, int64_t, int, int, hipStream_t) { return hit(); }
hipError_t launch_check(const CheckArgs&, hipStream_t) { return hit(); }
hipError_t launch_index_scores(const uint16_t*, const uint16_t*, const float*, float*, int, int, int, hipStream_t) {
  return hit();
}
hipError_t launch_select_tokens(const float*, int32_t*, int32_t*, int64_t, int, TopkParams, int, hipStream_t) {
  return hit();
}
hipError_t launch_select_marked(const float*, int32_t*, int32_t*, int64_t, int, TopkParams, int, hipStream_t) {
  return hit();
}
hipError_t launch_index_topk(const uint16_t*, const uint16_t*, const float*, int32_t*, int32_t*, void*, int, int, int,
                             TopkParams, int, hipStream_t) { return hit(); }
hipError_t launch_token_attn(const TokenAttnArgs&, int, hipStream_t) { return hit(); }
hipError_t launch_sparse_attn_fwd(const AttnArgs&, int, int, hipStream_t) { return hit(); }
hipError_t launch_bwd_prep(const uint16_t*, const uint16_t*, const float*, float*, int64_t, int, int, int, int,
                           hipStream_t) { return hit(); }
hipError_t launch_bwd_invert(const int32_t*, const int32_t*, int32_t*, int32_t*, int64_t, int, int, hipStream_t) {
  return hit();
}
hipError_t launch_sparse_attn_bwd(const BwdArgs&, int, int, hipStream_t) { return hit(); }
hipError_t launch_paged_decode(const PagedArgs&, int, int, TopkParams, hipStream_t) { return hit(); }
hipError_t launch_kv_append(const uint16_t*, const uint16_t*, const int32_t*, int32_t*, uint16_t*, uint16_t*, float*, int,
                            int, int, int, int, int, hipStream_t) { return hit(); }
hipError_t launch_paged_means(const uint16_t*, const int32_t*, const int32_t*, float*, int, int, int, int, int, int,
                              hipStream_t) { return hit(); }
hipError_t launch_paged_quantize(const uint16_t*, const uint16_t*, uint8_t*, uint8_t*, float*, float*, int, int, int, int,
                                 hipStream_t) { return hit(); }
hipError_t launch_kv_append_fp8(const uint16_t*, const uint16_t*, const int32_t*, int32_t*, uint8_t*, uint8_t*, float*,
                                float*, float*, int, int, int, int, int, int, hipStream_t) { return hit(); }
hipError_t launch_paged_means_fp8(const uint8_t*, const float*, const int32_t*, const int32_t*, float*, int, int, int, int,
                                  int, int, hipStream_t) { return hit(); }
hipError_t launch_decode(const DecodeArgs&, int, TopkParams, hipStream_t) { return hit(); }
static char fake_scratch[64];
hipError_t decode_noalloc_scratch(void** out) {
  *out = fake_scratch;
  return hit();
}
}  // namespace dsa
