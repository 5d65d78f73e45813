// Split-K paged decode over the int4 KIVI cache (gfx950), vector-ALU version.
//
// Method: S4 KV product page ("Funktionsweise" step 1): paged-attention KV
// cache stored as int4, KEY per channel, VALUE per token; the decode step is
// standard attention (header paragraph: head_dim 128, standard attention).
//
// One 64-lane work-group per (split, KV head, sequence). A split is a run of
// consecutive logical pages of one sequence; the last split of a sequence
// also takes the fp16 tail. Each work-group keeps an online softmax (running
// max m, running sum l, unnormalized output o) for the G query heads that
// share its KV head and writes (m, l, o) to the workspace; the reduce kernel
// merges the splits of a sequence into O.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include "internal.h"

namespace s4kv {
namespace {

constexpr float kNegInf = -INFINITY;

__device__ inline float nib(const uint8_t* base, int byte, int k) {
  return static_cast<float>((base[byte] >> (4 * (k & 1))) & 0xF);
}

// K code of (token t, channel d) inside a staged chunk (s4kv.h page format).
__device__ inline float k_code(const uint8_t* c, int t, int d) {
  const int m = d >> 5, g = (d & 31) >> 3, e = d & 7;
  const int kk = 4 * (e & 1) + (e >> 1);
  return nib(c + kOffKCodes, 16 * (16 * g + t) + 4 * m + (kk >> 1), kk);
}

// V code of (token t, channel d).
__device__ inline float v_code(const uint8_t* c, int t, int d) {
  const int tau = d >> 4, r = d & 15, g = t >> 2, j = t & 3;
  const int m = tau >> 1;
  const int kk = 4 * (j & 1) + 2 * (tau & 1) + (j >> 1);
  return nib(c + kOffVCodes, 16 * (16 * g + r) + 4 * m + (kk >> 1), kk);
}

template <int G>
__global__ __launch_bounds__(64) void decode_valu_kernel(
    const __half* __restrict__ q, const uint8_t* __restrict__ pages,
    const __half* __restrict__ tail_k, const __half* __restrict__ tail_v,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens, int32_t max_pages,
    int32_t hkv, int32_t pps, int32_t max_splits, float sm_scale, float* __restrict__ ws_o,
    float* __restrict__ ws_ml) {
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int hq = hkv * G;
  // ctx is clamped to what the block table and the launch can address, so a
  // broken precondition gives a wrong answer, never an out-of-bounds access.
  const int ctx = min(ctx_lens[b], max_pages * kPage);
  const int full = ctx > 0 ? ctx / kPage : 0;
  const int tail = ctx > 0 ? ctx % kPage : 0;
  const int nsplit = min(max_splits, max(1, (full + pps - 1) / pps));
  if (split >= nsplit) return;
  const int pbeg = split * pps;
  const int pend = (split == nsplit - 1) ? full : min(full, pbeg + pps);
  const bool do_tail = (split == nsplit - 1) && tail > 0;

  __shared__ float qs[G][kHeadDim];
  __shared__ __align__(16) uint8_t chunk[kChunkBytes];
  __shared__ float lg[G][kPage];

  for (int i = lane; i < G * kHeadDim; i += 64)
    qs[i / kHeadDim][i % kHeadDim] = __half2float(q[((int64_t)b * hq + h * G) * kHeadDim + i]);

  float m_run[G], l_run[G], o0[G], o1[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) { m_run[hh] = kNegInf; l_run[hh] = 0.f; o0[hh] = 0.f; o1[hh] = 0.f; }

  const int qt = lane & 15, qu = lane >> 4;  // QK mapping: token, channel quarter
  const int d0 = 2 * lane;                   // PV mapping: channel pair

  const int npg = (pend - pbeg) + (do_tail ? 1 : 0);
  for (int it = 0; it < npg; ++it) {
    const bool is_tail = (pbeg + it >= pend);
    const int ntok = is_tail ? tail : kPage;
    const __half* tk = tail_k + ((int64_t)b * hkv + h) * kPage * kHeadDim;
    const __half* tv = tail_v + ((int64_t)b * hkv + h) * kPage * kHeadDim;
    __syncthreads();
    if (!is_tail) {
      const uint8_t* src = pages + ((int64_t)block_table[(int64_t)b * max_pages + pbeg + it] * hkv + h) * kChunkStride;
      for (int i = lane; i < kChunkBytes / 16; i += 64)
        reinterpret_cast<uint4*>(chunk)[i] = reinterpret_cast<const uint4*>(src)[i];
    }
    __syncthreads();
    // ---- logits: lane (token qt, channels 32*qu .. +32) ----
    float acc[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) acc[hh] = 0.f;
    if (qt < ntok) {
      for (int i = 0; i < 32; ++i) {
        const int d = 32 * qu + i;
        float kh;
        if (is_tail) {
          kh = __half2float(tk[qt * kHeadDim + d]);
        } else {
          const float s = __half2float(reinterpret_cast<const __half*>(chunk + kOffKScale)[d]);
          const float z = __half2float(reinterpret_cast<const __half*>(chunk + kOffKZero)[d]);
          kh = k_code(chunk, qt, d) * s + z;
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) acc[hh] += qs[hh][d] * kh;
      }
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      acc[hh] += __shfl_xor(acc[hh], 16);
      acc[hh] += __shfl_xor(acc[hh], 32);
    }
    if (qu == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) lg[hh][qt] = (qt < ntok) ? acc[hh] * sm_scale : kNegInf;
    }
    __syncthreads();
    // ---- online softmax + PV: lane owns channels d0, d0+1 ----
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float pm = kNegInf;
      for (int t = 0; t < ntok; ++t) pm = fmaxf(pm, lg[hh][t]);
      const float mnew = fmaxf(m_run[hh], pm);
      const float alpha = (m_run[hh] == kNegInf) ? 0.f : expf(m_run[hh] - mnew);
      m_run[hh] = mnew;
      l_run[hh] *= alpha;
      o0[hh] *= alpha;
      o1[hh] *= alpha;
    }
    for (int t = 0; t < ntok; ++t) {
      float v0, v1;
      if (is_tail) {
        v0 = __half2float(tv[t * kHeadDim + d0]);
        v1 = __half2float(tv[t * kHeadDim + d0 + 1]);
      } else {
        const float s = __half2float(reinterpret_cast<const __half*>(chunk + kOffVScale)[t]);
        const float z = __half2float(reinterpret_cast<const __half*>(chunk + kOffVZero)[t]);
        v0 = v_code(chunk, t, d0) * s + z;
        v1 = v_code(chunk, t, d0 + 1) * s + z;
      }
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float p = expf(lg[hh][t] - m_run[hh]);
        l_run[hh] += p;
        o0[hh] += p * v0;
        o1[hh] += p * v1;
      }
    }
  }

#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const int64_t row = ((int64_t)b * hq + h * G + hh) * max_splits + split;
    reinterpret_cast<float2*>(ws_o + row * kHeadDim)[lane] = make_float2(o0[hh], o1[hh]);
    if (lane == 0) { ws_ml[2 * row] = m_run[hh]; ws_ml[2 * row + 1] = l_run[hh]; }
  }
}

// Merge the splits of (sequence, query head): M = max m_s,
// O = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s.
__global__ __launch_bounds__(128) void splitk_reduce_kernel(
    const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ ctx_lens, int32_t max_pages, int32_t hq, int32_t pps,
    int32_t max_splits, __half* __restrict__ out) {
  const int j = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int ctx = min(ctx_lens[b], max_pages * kPage);
  __half* o = out + ((int64_t)b * hq + j) * kHeadDim;
  if (ctx <= 0) { o[d] = __float2half(0.f); return; }
  const int full = ctx / kPage;
  const int nsplit = min(max_splits, max(1, (full + pps - 1) / pps));
  const int64_t row0 = ((int64_t)b * hq + j) * max_splits;
  float mx = kNegInf;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, ws_ml[2 * (row0 + s)]);
  float den = 0.f, num = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float ms = ws_ml[2 * (row0 + s)];
    const float w = (ms == kNegInf) ? 0.f : expf(ms - mx);
    den += w * ws_ml[2 * (row0 + s) + 1];
    num += w * ws_o[(row0 + s) * kHeadDim + d];
  }
  o[d] = __float2half_rn(num / den);
}

template <int G>
hipError_t launch_g(const s4kv_shape& s, const SplitPlan& plan, const void* q, const void* pages,
                    const void* tail_k, const void* tail_v, const int32_t* block_table,
                    const int32_t* ctx_lens, float sm_scale, float* ws_o, float* ws_ml,
                    hipStream_t stream) {
  dim3 grid(plan.max_splits, s.num_kv_heads, s.num_seqs);
  hipLaunchKernelGGL((decode_valu_kernel<G>), grid, dim3(64), 0, stream,
                     static_cast<const __half*>(q), static_cast<const uint8_t*>(pages),
                     static_cast<const __half*>(tail_k), static_cast<const __half*>(tail_v),
                     block_table, ctx_lens, s.max_pages_per_seq, s.num_kv_heads,
                     plan.pages_per_split, plan.max_splits, sm_scale, ws_o, ws_ml);
  return hipGetLastError();
}

}  // namespace

SplitPlan plan_splits(const s4kv_shape& s, int32_t max_ctx) {
  const int64_t max_full = max_ctx / kPage;
  // Aim for about 8192 work-groups over the whole batch when every sequence
  // is at max_ctx; never fewer than 8 pages per work-group.
  const int64_t work = (int64_t)s.num_seqs * s.num_kv_heads * max_full;
  int64_t pps = (work + 8191) / 8192;
  if (pps < 8) pps = 8;
  pps = (pps + 1) & ~int64_t(1);
  SplitPlan p;
  p.pages_per_split = static_cast<int>(pps);
  p.max_splits = static_cast<int>(max_full > 0 ? (max_full + pps - 1) / pps : 1);
  if (p.max_splits < 1) p.max_splits = 1;
  return p;
}

size_t workspace_bytes(const s4kv_shape& s, const SplitPlan& plan) {
  const size_t rows = (size_t)s.num_seqs * s.num_q_heads * plan.max_splits;
  size_t o_bytes = rows * kHeadDim * sizeof(float);
  o_bytes = (o_bytes + 255) & ~size_t(255);
  return o_bytes + rows * 2 * sizeof(float);
}

hipError_t launch_paged_decode(const s4kv_shape& s, const SplitPlan& plan, const void* q,
                               const void* pages, const void* tail_k, const void* tail_v,
                               const int32_t* block_table, const int32_t* ctx_lens,
                               float sm_scale, void* out, void* workspace, hipStream_t stream) {
  const size_t rows = (size_t)s.num_seqs * s.num_q_heads * plan.max_splits;
  size_t o_bytes = (rows * kHeadDim * sizeof(float) + 255) & ~size_t(255);
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  const int G = s.num_q_heads / s.num_kv_heads;
  hipError_t e = hipErrorInvalidValue;
  switch (G) {
#define S4KV_CASE(g) \
  case g: e = launch_g<g>(s, plan, q, pages, tail_k, tail_v, block_table, ctx_lens, sm_scale, ws_o, ws_ml, stream); break;
    S4KV_CASE(1) S4KV_CASE(2) S4KV_CASE(3) S4KV_CASE(4) S4KV_CASE(5) S4KV_CASE(6) S4KV_CASE(7)
    S4KV_CASE(8) S4KV_CASE(9) S4KV_CASE(10) S4KV_CASE(11) S4KV_CASE(12) S4KV_CASE(13)
    S4KV_CASE(14) S4KV_CASE(15) S4KV_CASE(16)
#undef S4KV_CASE
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3(s.num_q_heads, s.num_seqs), dim3(kHeadDim), 0,
                     stream, ws_o, ws_ml, ctx_lens, s.max_pages_per_seq, s.num_q_heads,
                     plan.pages_per_split,
                     plan.max_splits, static_cast<__half*>(out));
  return hipGetLastError();
}

}  // namespace s4kv
