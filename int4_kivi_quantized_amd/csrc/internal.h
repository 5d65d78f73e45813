// Internal declarations shared by the C-ABI layer and the HIP translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "s4kv.h"

namespace s4kv {

constexpr int kHeadDim = S4KV_HEAD_DIM;
constexpr int kPage = S4KV_PAGE_SIZE;
constexpr int kChunkBytes = S4KV_CHUNK_BYTES;
constexpr int kChunkStride = S4KV_CHUNK_STRIDE;
constexpr int kMaxGroup = S4KV_MAX_GROUP;

// Offsets inside a chunk (see s4kv.h, "Page format").
constexpr int kOffKCodes = 0;
constexpr int kOffVCodes = 1024;
constexpr int kOffKScale = 2048;
constexpr int kOffKZero = 2304;
constexpr int kOffVScale = 2560;
constexpr int kOffVZero = 2592;

// 2-bit KIVI pages (see s4kv.h, "2-bit KIVI pages").
constexpr int kK2ChunkBytes = S4KV_K2_CHUNK_BYTES;
constexpr int kK2ChunkStride = S4KV_K2_CHUNK_STRIDE;
constexpr int kOff2KCodes = 0;
constexpr int kOff2VCodes = 512;
constexpr int kOff2KScale = 1024;
constexpr int kOff2KZero = 1280;
constexpr int kOff2VScale = 1536;
constexpr int kOff2VZero = 1568;

// Decode workspace: the total unit count, the waves sharing each (sequence, head)
// and the per-(sequence, head, wave) partial results. The int4 and fp16 decode
// paths share it and the merge kernel.
size_t workspace_bytes(const s4kv_shape& s);

struct SplitWorkspace {
  int32_t* total_units;  // [0]: units of the launch, written by wave 0
  int32_t* seg_waves;    // [B * Hkv][2]: first / last wave sharing each (b, h)
  float* slots;          // partial results, G x (128 outputs, m, l, 2 pad) floats per slot
};
SplitWorkspace split_workspace(const s4kv_shape& s, void* workspace);

// Waves of the persistent decode grid: 8 per CU (two per SIMD).
int resident_waves();
// Upper bound on any persistent decode grid; the workspace holds partial-result
// slots for this many waves.
constexpr int kMaxWaves = 4096;

// Merge the partial results of a decode stream launched with W waves into
// fp16 out [B][Hq][128] (units per sequence: full pages plus one for a partial
// one, as both decode paths count them).
hipError_t launch_split_merge(const s4kv_shape& s, int W, int32_t max_ctx, const SplitWorkspace& ws,
                              const int32_t* ctx_lens, void* out, hipStream_t stream);

// bits: 4 (int4 pages) or 2 (2-bit KIVI pages)
hipError_t launch_quantize_append(const s4kv_shape& s, const void* k, const void* v,
                                  const int32_t* cu_new, const int32_t* slot, int32_t max_new,
                                  const int32_t* block_table, void* pages, void* tail_k,
                                  void* tail_v, hipStream_t stream, int bits = 4);

// Multi-query attention over the int4 cache: up to max_q query tokens per
// sequence, causal within the sequence. The (token, head) columns of a
// sequence go to the matrix cores in tiles of at most 16 columns (tpt whole
// tokens each); with more than one tile per sequence every tile is streamed
// as a virtual sequence of its own (ct_n tiles per sequence).
struct MqTiling {
  int32_t tpt;           // tokens per tile
  int32_t ct_n;          // tiles per sequence
  int32_t columns;       // columns per tile, tpt * Hq / Hkv
  int64_t virtual_seqs;  // num_seqs * ct_n
};
inline MqTiling mq_tiling(const s4kv_shape& s, int32_t max_q) {
  const int gq = s.num_q_heads / s.num_kv_heads;
  MqTiling t;
  if ((int64_t)max_q * gq <= kMaxGroup) {
    t.tpt = max_q;
    t.ct_n = 1;
  } else {
    t.tpt = kMaxGroup / gq;  // whole tokens per tile of at most 16 columns
    t.ct_n = static_cast<int32_t>(((int64_t)max_q + t.tpt - 1) / t.tpt);
  }
  t.columns = t.tpt * gq;
  t.virtual_seqs = (int64_t)s.num_seqs * t.ct_n;
  return t;
}
// Whether the tiles fit the launch limits: at most 65535 virtual sequences
// (the merge grid's y dimension) and a flat unit count that fits in int32.
inline bool mq_tiling_fits(const s4kv_shape& s, const MqTiling& t) {
  return t.virtual_seqs <= 65535 &&
         t.virtual_seqs * s.num_kv_heads * ((int64_t)s.max_pages_per_seq + 1) <= INT32_MAX;
}
size_t mq_workspace_bytes(const s4kv_shape& s, int32_t max_q);
// Append one token per sequence (position ctx_lens[b] - 1, from k_new /
// v_new [B][Hkv][128]) and decode, in one launch of the decode stream.
hipError_t launch_paged_decode_append(const s4kv_shape& s, const void* q, const void* k_new,
                                      const void* v_new, void* pages, void* tail_k, void* tail_v,
                                      const int32_t* block_table, const int32_t* ctx_lens,
                                      int32_t max_ctx, float sm_scale, void* out, void* workspace,
                                      hipStream_t stream);
// The same with the workspace in the library's static per-device array
// (S4KV_NOALLOC_SCRATCH_BYTES; the caller has checked the size).
hipError_t launch_paged_decode_append_noalloc(const s4kv_shape& s, const void* q, const void* k_new,
                                              const void* v_new, void* pages, void* tail_k,
                                              void* tail_v, const int32_t* block_table,
                                              const int32_t* ctx_lens, int32_t max_ctx,
                                              float sm_scale, void* out, hipStream_t stream);
hipError_t launch_paged_mq(const s4kv_shape& s, const void* q, const int32_t* cu_q, int32_t max_q,
                           int32_t total_q, const void* pages, const void* tail_k, const void* tail_v,
                           const int32_t* block_table, const int32_t* ctx_lens, int32_t max_ctx,
                           float sm_scale, void* out, void* workspace, hipStream_t stream);

// bits: 4 (int4 pages) or 2 (2-bit KIVI pages)
hipError_t launch_paged_decode(const s4kv_shape& s, const void* q,
                               const void* pages, const void* tail_k, const void* tail_v,
                               const int32_t* block_table, const int32_t* ctx_lens,
                               int32_t max_ctx, float sm_scale, void* out, void* workspace,
                               hipStream_t stream, int bits = 4);

// Dense paged caches (dense_decode.hip): fp16 control path and FP8 E4M3.
constexpr int kF16ChunkHalves = 2 * S4KV_PAGE_SIZE * S4KV_HEAD_DIM;  // K block, then V^T block
hipError_t launch_fp16_append(const s4kv_shape& s, const void* k, const void* v,
                              const int32_t* cu_new, const int32_t* slot, int32_t max_new,
                              const int32_t* block_table, void* pages, hipStream_t stream);
hipError_t launch_fp16_decode(const s4kv_shape& s, const void* q, const void* pages,
                              const int32_t* block_table, const int32_t* ctx_lens, int32_t max_ctx,
                              float sm_scale, void* out, void* workspace, hipStream_t stream);
constexpr int kF8ChunkBytes = S4KV_FP8_CHUNK_BYTES;  // K blocks, then V blocks, operand order
hipError_t launch_fp8_append(const s4kv_shape& s, const void* k, const void* v, const int32_t* cu_new,
                             const int32_t* slot, int32_t max_new, const int32_t* block_table,
                             const float* k_scale, const float* v_scale, void* pages, hipStream_t stream);
hipError_t launch_fp8_decode(const s4kv_shape& s, const void* q, const void* pages,
                             const int32_t* block_table, const int32_t* ctx_lens, int32_t max_ctx,
                             float sm_scale, const float* k_scale, const float* v_scale, void* out,
                             void* workspace, hipStream_t stream);

// Table checks (check_tables.hip): report int32 [4] as s4kv_check_tables.
hipError_t launch_check_tables(const s4kv_shape& s, const int32_t* block_table,
                               const int32_t* ctx_lens, int32_t max_ctx, int32_t* report,
                               hipStream_t stream);

}  // namespace s4kv
