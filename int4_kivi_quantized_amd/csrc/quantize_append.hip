// Quantize-on-append for the int4 KIVI paged cache (gfx950).
//
// Method: S4 KV product page ("Funktionsweise" step 1): asymmetric int4, KEY
// per channel, VALUE per token. A page is quantized once, when its 16th token
// arrives; until then its tokens stay fp16 in the per-sequence tail.
//
// One 64-lane wave per (sequence, KV head, page touched by the append). The
// same kernel serves a decode step (one token per sequence) and a bulk
// prefill (thousands of tokens per sequence): full pages are quantized
// straight from the input rows, only the first page can take older tokens
// from the tail, and only the last page can leave tokens in the tail.
//
// Rounding is fixed so that codes are reproducible bit for bit: IEEE fp32
// subtract and correctly rounded divide (HIP's default division), round half
// to even, clamp to [0, 15]; no contraction into fused multiply-adds.
//
// The same kernel, instantiated for 2-bit codes, fills the 2-bit KIVI pages
// (the KIVI paper cited by the KV-cache explainer, analyticslegends.ai,
// "Quellen", entry 17): scale (max - min) / 3, codes 0..3, the page layout of
// s4kv.h's 2-bit section.
#pragma clang fp contract(off)

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "internal.h"
#include "page_quant.h"

namespace s4kv {
namespace {

__device__ inline const __half* token_row(int pos, int start, int64_t in_row0, int h, int hkv,
                                          const __half* in, const __half* tail) {
  // row of 128 fp16 for position `pos` of this (sequence, head)
  if (pos < start) return tail + (pos & (kPage - 1)) * kHeadDim;
  return in + ((in_row0 + (pos - start)) * hkv + h) * kHeadDim;
}

template <int kBits>
__global__ __launch_bounds__(64) void quantize_append_kernel(
    const __half* __restrict__ k, const __half* __restrict__ v, const int32_t* __restrict__ cu_new,
    const int32_t* __restrict__ slot, const int32_t* __restrict__ block_table, int32_t max_pages,
    uint8_t* __restrict__ pages, __half* tail_k, __half* tail_v, int32_t hkv) {
  const int x = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x;

  const int start = slot[b];
  const int64_t in_row0 = cu_new[b];
  const int n = cu_new[b + 1] - cu_new[b];
  if (n <= 0) return;
  const int end = start + n;
  const int p0 = start / kPage;
  const int plast = (end - 1) / kPage;
  const int p = p0 + x;
  if (p > plast) return;

  __half* tk = tail_k + ((int64_t)b * hkv + h) * kPage * kHeadDim;
  __half* tv = tail_v + ((int64_t)b * hkv + h) * kPage * kHeadDim;

  __shared__ uint8_t kc[kPage][kHeadDim];
  __shared__ uint8_t vc[kPage][kHeadDim];

  using C = Codes<kBits>;
  if ((p + 1) * kPage <= end) {
    // ---- the page is full: quantize its 16 tokens ----
    uint8_t* chunk = pages + ((int64_t)block_table[(int64_t)b * max_pages + p] * hkv + h) * C::kStride;

    // K and V rows of page token t: input rows from `start` on, tail rows before
    const int base = p * kPage;
    auto krow = [&](int t) { return token_row(base + t, start, in_row0, h, hkv, k, tk); };
    auto vrow = [&](int t) { return token_row(base + t, start, in_row0, h, hkv, v, tv); };
    PageShare<kBits> share;
    // scales and zeros go out while the rest of the page is computed
    quantize_page<kBits>(krow, vrow, lane, kc, vc, share,
                         [&](const PageShare<kBits>& sh) { store_page_kmeta<kBits>(chunk, lane, sh); },
                         [&](const PageShare<kBits>& sh) { store_page_vmeta<kBits>(chunk, lane, sh, true); });
    store_page_codes<kBits>(chunk, lane, share);
  }

  if (x == 0 && (end % kPage) != 0) {
    // The first wave of the sequence also stores the new tokens of the last,
    // partial page into the tail -- after its own flush has read the old tail
    // tokens, so the two never race.
    __syncthreads();
    const int first = max(start, plast * kPage);
    for (int pos = first; pos < end; ++pos) {
      const int64_t row = ((in_row0 + (pos - start)) * hkv + h) * kHeadDim;
      const int ts = (pos & (kPage - 1)) * kHeadDim;
      reinterpret_cast<__half2*>(tk + ts)[lane] = reinterpret_cast<const __half2*>(k + row)[lane];
      reinterpret_cast<__half2*>(tv + ts)[lane] = reinterpret_cast<const __half2*>(v + row)[lane];
    }
  }
}

}  // namespace

hipError_t launch_quantize_append(const s4kv_shape& s, const void* k, const void* v,
                                  const int32_t* cu_new, const int32_t* slot, int32_t max_new,
                                  const int32_t* block_table, void* pages, void* tail_k,
                                  void* tail_v, hipStream_t stream, int bits) {
  // pages touched by n tokens starting anywhere inside a page: floor((n+14)/16)+1
  const int slots = (max_new + 14) / kPage + 1;
  dim3 grid(slots, s.num_kv_heads, s.num_seqs);
  if (bits == 2) {
    hipLaunchKernelGGL(quantize_append_kernel<2>, grid, dim3(64), 0, stream,
                       static_cast<const __half*>(k), static_cast<const __half*>(v), cu_new, slot,
                       block_table, s.max_pages_per_seq, static_cast<uint8_t*>(pages),
                       static_cast<__half*>(tail_k), static_cast<__half*>(tail_v), s.num_kv_heads);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(quantize_append_kernel<4>, grid, dim3(64), 0, stream,
                     static_cast<const __half*>(k), static_cast<const __half*>(v), cu_new, slot,
                     block_table, s.max_pages_per_seq, static_cast<uint8_t*>(pages),
                     static_cast<__half*>(tail_k), static_cast<__half*>(tail_v), s.num_kv_heads);
  return hipGetLastError();
}

}  // namespace s4kv
