// C ABI of the s4kv library: host-side validation and dispatch.
//
// Fail-fast validation follows the S4 KV product page ("Highlights", "FAQ"):
// only head_dim 128 with standard attention is supported, and anything else is
// refused before any work is done rather than producing wrong output.
#include <hip/hip_runtime_api.h>

#include "internal.h"

namespace {

s4kv_status check_shape(const s4kv_shape* s) {
  if (s == nullptr) return S4KV_ERR_INVALID_ARG;
  if (s->num_seqs < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->num_pages < 1 ||
      s->max_pages_per_seq < 1)
    return S4KV_ERR_INVALID_ARG;
  if (s->head_dim != S4KV_HEAD_DIM || s->page_size != S4KV_PAGE_SIZE) return S4KV_ERR_UNSUPPORTED;
  if (s->num_q_heads % s->num_kv_heads != 0) return S4KV_ERR_UNSUPPORTED;
  if (s->num_q_heads / s->num_kv_heads > S4KV_MAX_GROUP) return S4KV_ERR_UNSUPPORTED;
  // launch-grid limits (y and z dimensions)
  if (s->num_kv_heads > 65535 || s->num_seqs > 65535 || s->num_q_heads > 65535)
    return S4KV_ERR_UNSUPPORTED;
  // chunk indices (page * Hkv + head) must fit in int32
  if ((int64_t)s->num_pages * s->num_kv_heads > INT32_MAX) return S4KV_ERR_INVALID_ARG;
  // token positions and the flat unit count (B * Hkv * (pages + 1)) must fit in int32
  if ((int64_t)s->max_pages_per_seq * S4KV_PAGE_SIZE > INT32_MAX) return S4KV_ERR_INVALID_ARG;
  if ((int64_t)s->num_seqs * s->num_kv_heads * ((int64_t)s->max_pages_per_seq + 1) > INT32_MAX)
    return S4KV_ERR_INVALID_ARG;
  return S4KV_OK;
}

}  // namespace

extern "C" {

s4kv_status s4kv_validate(const s4kv_shape* shape) { return check_shape(shape); }

const char* s4kv_status_string(s4kv_status status) {
  switch (status) {
    case S4KV_OK: return "ok";
    case S4KV_ERR_INVALID_ARG: return "invalid argument";
    case S4KV_ERR_UNSUPPORTED: return "unsupported shape (needs head_dim 128, page 16, Hq % Hkv == 0, Hq/Hkv <= 16)";
    case S4KV_ERR_WORKSPACE: return "workspace too small";
    case S4KV_ERR_HIP: return "HIP launch failed";
    case S4KV_ERR_SCRATCH_LIMIT:
      return "shape needs more decode workspace than the static scratch (S4KV_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

size_t s4kv_pool_bytes(const s4kv_shape* shape) {
  if (check_shape(shape) != S4KV_OK) return 0;
  return (size_t)shape->num_pages * shape->num_kv_heads * S4KV_CHUNK_STRIDE;
}

size_t s4kv_tail_bytes(const s4kv_shape* shape) {
  if (check_shape(shape) != S4KV_OK) return 0;
  return (size_t)shape->num_seqs * shape->num_kv_heads * S4KV_PAGE_SIZE * S4KV_HEAD_DIM * 2;
}

s4kv_status s4kv_quantize_append(const s4kv_shape* shape, const void* k, const void* v,
                                 const int32_t* cu_new, const int32_t* slot, int32_t max_new,
                                 const int32_t* block_table, void* pages, void* tail_k,
                                 void* tail_v, void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (max_new < 0) return S4KV_ERR_INVALID_ARG;
  if (!k || !v || !cu_new || !slot || !block_table || !pages || !tail_k || !tail_v)
    return S4KV_ERR_INVALID_ARG;
  if (max_new == 0) return S4KV_OK;
  if ((int64_t)max_new > (int64_t)shape->max_pages_per_seq * S4KV_PAGE_SIZE)
    return S4KV_ERR_INVALID_ARG;
  const hipError_t e = s4kv::launch_quantize_append(*shape, k, v, cu_new, slot, max_new,
                                                    block_table, pages, tail_k, tail_v,
                                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

s4kv_status s4kv_check_tables(const s4kv_shape* shape, const int32_t* block_table,
                              const int32_t* ctx_lens, int32_t max_ctx, int32_t* report,
                              void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (!block_table || !ctx_lens || !report || max_ctx < 0) return S4KV_ERR_INVALID_ARG;
  const hipError_t e = s4kv::launch_check_tables(*shape, block_table, ctx_lens, max_ctx, report,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

size_t s4kv_decode_workspace_bytes(const s4kv_shape* shape, int32_t max_ctx) {
  if (check_shape(shape) != S4KV_OK || max_ctx < 1) return 0;
  return s4kv::workspace_bytes(*shape);
}

s4kv_status s4kv_paged_decode(const s4kv_shape* shape, const void* q, const void* pages,
                              const void* tail_k, const void* tail_v,
                              const int32_t* block_table, const int32_t* ctx_lens,
                              int32_t max_ctx, float sm_scale, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (max_ctx < 1 || (int64_t)max_ctx > (int64_t)shape->max_pages_per_seq * S4KV_PAGE_SIZE)
    return S4KV_ERR_INVALID_ARG;
  if (!q || !pages || !tail_k || !tail_v || !block_table || !ctx_lens || !out || !workspace)
    return S4KV_ERR_INVALID_ARG;
  if (workspace_bytes < s4kv::workspace_bytes(*shape)) return S4KV_ERR_WORKSPACE;
  const hipError_t e = s4kv::launch_paged_decode(*shape, q, pages, tail_k, tail_v,
                                                 block_table, ctx_lens, max_ctx, sm_scale, out, workspace,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

s4kv_status s4kv_paged_decode_append(const s4kv_shape* shape, const void* q, const void* k_new,
                                     const void* v_new, void* pages, void* tail_k, void* tail_v,
                                     const int32_t* block_table, const int32_t* ctx_lens,
                                     int32_t max_ctx, float sm_scale, void* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (max_ctx < 1 || (int64_t)max_ctx > (int64_t)shape->max_pages_per_seq * S4KV_PAGE_SIZE)
    return S4KV_ERR_INVALID_ARG;
  if (!q || !k_new || !v_new || !pages || !tail_k || !tail_v || !block_table || !ctx_lens || !out ||
      !workspace)
    return S4KV_ERR_INVALID_ARG;
  if (workspace_bytes < s4kv::workspace_bytes(*shape)) return S4KV_ERR_WORKSPACE;
  const hipError_t e = s4kv::launch_paged_decode_append(*shape, q, k_new, v_new, pages, tail_k,
                                                        tail_v, block_table, ctx_lens, max_ctx,
                                                        sm_scale, out, workspace,
                                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

s4kv_status s4kv_paged_decode_append_noalloc(const s4kv_shape* shape, const void* q,
                                             const void* k_new, const void* v_new, void* pages,
                                             void* tail_k, void* tail_v,
                                             const int32_t* block_table, const int32_t* ctx_lens,
                                             int32_t max_ctx, float sm_scale, void* out,
                                             void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (max_ctx < 1 || (int64_t)max_ctx > (int64_t)shape->max_pages_per_seq * S4KV_PAGE_SIZE)
    return S4KV_ERR_INVALID_ARG;
  if (!q || !k_new || !v_new || !pages || !tail_k || !tail_v || !block_table || !ctx_lens || !out)
    return S4KV_ERR_INVALID_ARG;
  if (s4kv::workspace_bytes(*shape) > (size_t)S4KV_NOALLOC_SCRATCH_BYTES)
    return S4KV_ERR_SCRATCH_LIMIT;
  const hipError_t e = s4kv::launch_paged_decode_append_noalloc(
      *shape, q, k_new, v_new, pages, tail_k, tail_v, block_table, ctx_lens, max_ctx, sm_scale,
      out, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

size_t s4kv_kivi2_pool_bytes(const s4kv_shape* shape) {
  if (check_shape(shape) != S4KV_OK) return 0;
  return (size_t)shape->num_pages * shape->num_kv_heads * S4KV_K2_CHUNK_STRIDE;
}

s4kv_status s4kv_kivi2_quantize_append(const s4kv_shape* shape, const void* k, const void* v,
                                       const int32_t* cu_new, const int32_t* slot,
                                       int32_t max_new, const int32_t* block_table, void* pages,
                                       void* tail_k, void* tail_v, void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (max_new < 0) return S4KV_ERR_INVALID_ARG;
  if (!k || !v || !cu_new || !slot || !block_table || !pages || !tail_k || !tail_v)
    return S4KV_ERR_INVALID_ARG;
  if (max_new == 0) return S4KV_OK;
  if ((int64_t)max_new > (int64_t)shape->max_pages_per_seq * S4KV_PAGE_SIZE)
    return S4KV_ERR_INVALID_ARG;
  const hipError_t e = s4kv::launch_quantize_append(*shape, k, v, cu_new, slot, max_new,
                                                    block_table, pages, tail_k, tail_v,
                                                    static_cast<hipStream_t>(stream), 2);
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

s4kv_status s4kv_kivi2_paged_decode(const s4kv_shape* shape, const void* q, const void* pages,
                                    const void* tail_k, const void* tail_v,
                                    const int32_t* block_table, const int32_t* ctx_lens,
                                    int32_t max_ctx, float sm_scale, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (max_ctx < 1 || (int64_t)max_ctx > (int64_t)shape->max_pages_per_seq * S4KV_PAGE_SIZE)
    return S4KV_ERR_INVALID_ARG;
  if (!q || !pages || !tail_k || !tail_v || !block_table || !ctx_lens || !out || !workspace)
    return S4KV_ERR_INVALID_ARG;
  if (workspace_bytes < s4kv::workspace_bytes(*shape)) return S4KV_ERR_WORKSPACE;
  const hipError_t e = s4kv::launch_paged_decode(*shape, q, pages, tail_k, tail_v, block_table,
                                                 ctx_lens, max_ctx, sm_scale, out, workspace,
                                                 static_cast<hipStream_t>(stream), 2);
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

size_t s4kv_mq_workspace_bytes(const s4kv_shape* shape, int32_t max_ctx, int32_t max_q) {
  if (check_shape(shape) != S4KV_OK || max_ctx < 1 || max_q < 1) return 0;
  if (!s4kv::mq_tiling_fits(*shape, s4kv::mq_tiling(*shape, max_q))) return 0;
  return s4kv::mq_workspace_bytes(*shape, max_q);
}

s4kv_status s4kv_paged_attention_mq(const s4kv_shape* shape, const void* q, const int32_t* cu_q,
                                    int32_t max_q, int32_t total_q, const void* pages,
                                    const void* tail_k, const void* tail_v,
                                    const int32_t* block_table, const int32_t* ctx_lens,
                                    int32_t max_ctx, float sm_scale, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (max_ctx < 1 || (int64_t)max_ctx > (int64_t)shape->max_pages_per_seq * S4KV_PAGE_SIZE)
    return S4KV_ERR_INVALID_ARG;
  if (max_q < 1 || total_q < 1) return S4KV_ERR_INVALID_ARG;
  if (!s4kv::mq_tiling_fits(*shape, s4kv::mq_tiling(*shape, max_q))) return S4KV_ERR_UNSUPPORTED;
  // query rows times heads must index in int64 without overflow of int32 row counts
  if ((int64_t)total_q > (int64_t)shape->num_seqs * max_q) return S4KV_ERR_INVALID_ARG;
  if (!q || !cu_q || !pages || !tail_k || !tail_v || !block_table || !ctx_lens || !out || !workspace)
    return S4KV_ERR_INVALID_ARG;
  if (workspace_bytes < s4kv::mq_workspace_bytes(*shape, max_q)) return S4KV_ERR_WORKSPACE;
  const hipError_t e = s4kv::launch_paged_mq(*shape, q, cu_q, max_q, total_q, pages, tail_k, tail_v,
                                             block_table, ctx_lens, max_ctx, sm_scale, out, workspace,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

size_t s4kv_fp16_pool_bytes(const s4kv_shape* shape) {
  if (check_shape(shape) != S4KV_OK) return 0;
  return (size_t)shape->num_pages * shape->num_kv_heads * S4KV_F16_CHUNK_BYTES;
}

s4kv_status s4kv_fp16_append(const s4kv_shape* shape, const void* k, const void* v,
                             const int32_t* cu_new, const int32_t* slot, int32_t max_new,
                             const int32_t* block_table, void* pages, void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (max_new < 0) return S4KV_ERR_INVALID_ARG;
  if (!k || !v || !cu_new || !slot || !block_table || !pages) return S4KV_ERR_INVALID_ARG;
  if (max_new == 0) return S4KV_OK;
  if ((int64_t)max_new > (int64_t)shape->max_pages_per_seq * S4KV_PAGE_SIZE)
    return S4KV_ERR_INVALID_ARG;
  const hipError_t e = s4kv::launch_fp16_append(*shape, k, v, cu_new, slot, max_new, block_table,
                                                pages, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

s4kv_status s4kv_fp16_paged_decode(const s4kv_shape* shape, const void* q, const void* pages,
                                   const int32_t* block_table, const int32_t* ctx_lens,
                                   int32_t max_ctx, float sm_scale, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (max_ctx < 1 || (int64_t)max_ctx > (int64_t)shape->max_pages_per_seq * S4KV_PAGE_SIZE)
    return S4KV_ERR_INVALID_ARG;
  if (!q || !pages || !block_table || !ctx_lens || !out || !workspace) return S4KV_ERR_INVALID_ARG;
  if (workspace_bytes < s4kv::workspace_bytes(*shape)) return S4KV_ERR_WORKSPACE;
  const hipError_t e = s4kv::launch_fp16_decode(*shape, q, pages, block_table, ctx_lens, max_ctx,
                                                sm_scale, out, workspace,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

size_t s4kv_fp8_pool_bytes(const s4kv_shape* shape) {
  if (check_shape(shape) != S4KV_OK) return 0;
  return (size_t)shape->num_pages * shape->num_kv_heads * S4KV_FP8_CHUNK_BYTES;
}

s4kv_status s4kv_fp8_append(const s4kv_shape* shape, const void* k, const void* v,
                            const int32_t* cu_new, const int32_t* slot, int32_t max_new,
                            const int32_t* block_table, const float* k_scale,
                            const float* v_scale, void* pages, void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (max_new < 0) return S4KV_ERR_INVALID_ARG;
  if (!k || !v || !cu_new || !slot || !block_table || !k_scale || !v_scale || !pages)
    return S4KV_ERR_INVALID_ARG;
  if (max_new == 0) return S4KV_OK;
  if ((int64_t)max_new > (int64_t)shape->max_pages_per_seq * S4KV_PAGE_SIZE)
    return S4KV_ERR_INVALID_ARG;
  const hipError_t e = s4kv::launch_fp8_append(*shape, k, v, cu_new, slot, max_new, block_table,
                                               k_scale, v_scale, pages,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

s4kv_status s4kv_fp8_paged_decode(const s4kv_shape* shape, const void* q, const void* pages,
                                  const int32_t* block_table, const int32_t* ctx_lens,
                                  int32_t max_ctx, float sm_scale, const float* k_scale,
                                  const float* v_scale, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  const s4kv_status st = check_shape(shape);
  if (st != S4KV_OK) return st;
  if (max_ctx < 1 || (int64_t)max_ctx > (int64_t)shape->max_pages_per_seq * S4KV_PAGE_SIZE)
    return S4KV_ERR_INVALID_ARG;
  if (!q || !pages || !block_table || !ctx_lens || !k_scale || !v_scale || !out || !workspace)
    return S4KV_ERR_INVALID_ARG;
  if (workspace_bytes < s4kv::workspace_bytes(*shape)) return S4KV_ERR_WORKSPACE;
  const hipError_t e = s4kv::launch_fp8_decode(*shape, q, pages, block_table, ctx_lens, max_ctx,
                                               sm_scale, k_scale, v_scale, out, workspace,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? S4KV_OK : S4KV_ERR_HIP;
}

}  // extern "C"
