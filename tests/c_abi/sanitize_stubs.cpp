// Stand-ins for the library's kernel launchers and workspace sizes, so that
// the C-ABI layer (csrc/api.cpp: shape validation, argument checks, dispatch)
// can be built and driven on the host alone, under AddressSanitizer and
// UndefinedBehaviorSanitizer. Each launcher only records that it was reached.
#include "internal.h"

namespace {
int g_launches = 0;
}

extern "C" int stub_launches(void) { return g_launches; }

namespace s4kv {

size_t workspace_bytes(const s4kv_shape& s) {
  return 4096 + (size_t)s.num_seqs * s.num_kv_heads * 64;
}
size_t mq_workspace_bytes(const s4kv_shape& s, int32_t max_q) {
  return workspace_bytes(s) * (size_t)mq_tiling(s, max_q).ct_n * 2;
}
hipError_t launch_check_tables(const s4kv_shape&, const int32_t*, const int32_t*, int32_t, int32_t*,
                               hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_quantize_append(const s4kv_shape&, const void*, const void*, const int32_t*,
                                  const int32_t*, int32_t, const int32_t*, void*, void*, void*,
                                  hipStream_t, int) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_paged_decode_append(const s4kv_shape&, const void*, const void*, const void*,
                                      void*, void*, void*, const int32_t*, const int32_t*,
                                      int32_t, float, void*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_paged_decode_append_noalloc(const s4kv_shape&, const void*, const void*,
                                              const void*, void*, void*, void*, const int32_t*,
                                              const int32_t*, int32_t, float, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_paged_mq(const s4kv_shape&, const void*, const int32_t*, int32_t, int32_t,
                           const void*, const void*, const void*, const int32_t*, const int32_t*,
                           int32_t, float, void*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_paged_decode(const s4kv_shape&, const void*, const void*, const void*,
                               const void*, const int32_t*, const int32_t*, int32_t, float, void*,
                               void*, hipStream_t, int) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fp16_append(const s4kv_shape&, const void*, const void*, const int32_t*,
                              const int32_t*, int32_t, const int32_t*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fp16_decode(const s4kv_shape&, const void*, const void*, const int32_t*,
                              const int32_t*, int32_t, float, void*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fp8_append(const s4kv_shape&, const void*, const void*, const int32_t*,
                             const int32_t*, int32_t, const int32_t*, const float*, const float*,
                             void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fp8_decode(const s4kv_shape&, const void*, const void*, const int32_t*,
                             const int32_t*, int32_t, float, const float*, const float*, void*,
                             void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

}  // namespace s4kv
