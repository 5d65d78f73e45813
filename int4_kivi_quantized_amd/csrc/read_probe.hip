// Streaming-read probe (a measurement aid, see s4kv_probe.h): the decode
// kernels' chunk loads with nothing else attached.
#include <hip/hip_runtime.h>

#include "s4kv_probe.h"

namespace {

constexpr int kChunk = S4KV_PROBE_CHUNK_BYTES;

template <int Aux>
__global__ __launch_bounds__(64) void probe_read_kernel(const uint8_t* __restrict__ pool,
                                                        uint64_t pool_bytes,
                                                        const int32_t* __restrict__ ids, int n) {
  __shared__ __align__(16) uint8_t sink[1024];
  const int lane = threadIdx.x;
  const int32_t* my = ids + (int64_t)blockIdx.x * n;
  for (int i = 0; i < n; ++i) {
    const int id = __builtin_amdgcn_readfirstlane(my[i]);
    if (id < 0 || ((uint64_t)id + 1) * kChunk > pool_bytes) continue;
    const uint8_t* src = pool + (uint64_t)id * kChunk + 16 * lane;
#pragma unroll
    for (int k = 0; k < kChunk / 1024; ++k)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + 1024 * k),
                                       (__attribute__((address_space(3))) void*)(sink), 16, 0, Aux);
    // vmcnt(0) only (gfx9 encoding): the chunk has landed before the next is issued
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
  }
}

}  // namespace

extern "C" s4kv_status s4kv_probe_read(const void* pool, size_t pool_bytes, const int32_t* chunk_ids,
                                       int32_t chunks_per_wave, int32_t waves, int32_t non_temporal,
                                       void* stream) {
  if (!pool || !chunk_ids || pool_bytes < (size_t)kChunk || chunks_per_wave < 1 || waves < 1)
    return S4KV_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* p = static_cast<const uint8_t*>(pool);
  if (non_temporal)
    hipLaunchKernelGGL(probe_read_kernel<2>, dim3(waves), dim3(64), 0, st, p, (uint64_t)pool_bytes,
                       chunk_ids, chunks_per_wave);
  else
    hipLaunchKernelGGL(probe_read_kernel<0>, dim3(waves), dim3(64), 0, st, p, (uint64_t)pool_bytes,
                       chunk_ids, chunks_per_wave);
  return hipGetLastError() == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}
