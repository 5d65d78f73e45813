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

namespace s4kv {
namespace {

// Code width: page geometry and the largest code.
template <int kBits>
struct Codes;
template <>
struct Codes<4> {
  static constexpr float kQmax = 15.0f;
  static constexpr int kStride = kChunkStride, kData = kChunkBytes;
  static constexpr int kK = kOffKCodes, kV = kOffVCodes, kKs = kOffKScale, kKz = kOffKZero,
                       kVs = kOffVScale, kVz = kOffVZero;
};
template <>
struct Codes<2> {
  static constexpr float kQmax = 3.0f;
  static constexpr int kStride = kK2ChunkStride, kData = kK2ChunkBytes;
  static constexpr int kK = kOff2KCodes, kV = kOff2VCodes, kKs = kOff2KScale, kKz = kOff2KZero,
                       kVs = kOff2VScale, kVz = kOff2VZero;
};

struct GroupQ {
  __half s;
  __half z;
  float sf;  // s as float (0 when codes are all 0)
  float zf;
};

// Scale/zero of a group from its fp32 min and max (both exact fp16 values).
template <int kBits>
__device__ inline GroupQ group_params(float mn, float mx) {
  GroupQ g;
  const float s32 = (mx - mn) / Codes<kBits>::kQmax;
  g.s = __float2half_rn(s32);
  g.z = __float2half_rn(mn);
  g.sf = __half2float(g.s);
  g.zf = __half2float(g.z);
  if (g.sf == 0.0f) { g.s = __ushort_as_half(0); g.sf = 0.0f; }
  if (g.zf == 0.0f) { g.z = __ushort_as_half(0); g.zf = 0.0f; }
  return g;
}

template <int kBits>
__device__ inline uint32_t code_of(float x, const GroupQ& g) {
  if (g.sf == 0.0f) return 0u;
  float t = rintf((x - g.zf) / g.sf);
  t = fminf(fmaxf(t, 0.0f), Codes<kBits>::kQmax);
  return static_cast<uint32_t>(t);
}

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

    // K: lane owns channels 2*lane, 2*lane+1; groups run over the 16 tokens.
    float k0[kPage], k1[kPage];
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      const __half* row = token_row(p * kPage + t, start, in_row0, h, hkv, k, tk);
      const __half2 v2 = reinterpret_cast<const __half2*>(row)[lane];
      k0[t] = __low2float(v2);
      k1[t] = __high2float(v2);
    }
    float mn0 = k0[0], mx0 = k0[0], mn1 = k1[0], mx1 = k1[0];
#pragma unroll
    for (int t = 1; t < kPage; ++t) {
      mn0 = fminf(mn0, k0[t]); mx0 = fmaxf(mx0, k0[t]);
      mn1 = fminf(mn1, k1[t]); mx1 = fmaxf(mx1, k1[t]);
    }
    const GroupQ g0 = group_params<kBits>(mn0, mx0);
    const GroupQ g1 = group_params<kBits>(mn1, mx1);
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      kc[t][2 * lane] = static_cast<uint8_t>(code_of<kBits>(k0[t], g0));
      kc[t][2 * lane + 1] = static_cast<uint8_t>(code_of<kBits>(k1[t], g1));
    }
    reinterpret_cast<__half2*>(chunk + C::kKs)[lane] = __halves2half2(g0.s, g1.s);
    reinterpret_cast<__half2*>(chunk + C::kKz)[lane] = __halves2half2(g0.z, g1.z);

    // V: lane owns token t = lane/4, channels 32*(lane%4) .. +32; groups run
    // over the token's 128 channels (4 lanes per token).
    const int vt = lane >> 2, vu = lane & 3;
    const __half* vrow = token_row(p * kPage + vt, start, in_row0, h, hkv, v, tv) + 32 * vu;
    float vx[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = reinterpret_cast<const uint4*>(vrow)[i];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const __half2 h2 = *reinterpret_cast<const __half2*>(&ws[j]);
        vx[8 * i + 2 * j] = __low2float(h2);
        vx[8 * i + 2 * j + 1] = __high2float(h2);
      }
    }
    float vmn = vx[0], vmx = vx[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) { vmn = fminf(vmn, vx[i]); vmx = fmaxf(vmx, vx[i]); }
    vmn = fminf(vmn, __shfl_xor(vmn, 1)); vmx = fmaxf(vmx, __shfl_xor(vmx, 1));
    vmn = fminf(vmn, __shfl_xor(vmn, 2)); vmx = fmaxf(vmx, __shfl_xor(vmx, 2));
    const GroupQ gv = group_params<kBits>(vmn, vmx);
#pragma unroll
    for (int i = 0; i < 32; ++i) vc[vt][32 * vu + i] = static_cast<uint8_t>(code_of<kBits>(vx[i], gv));
    if (vu == 0) {
      reinterpret_cast<__half*>(chunk + C::kVs)[vt] = gv.s;
      reinterpret_cast<__half*>(chunk + C::kVz)[vt] = gv.z;
    }
    // the 64 padding bytes after the data
    if (lane < 16) reinterpret_cast<uint32_t*>(chunk + C::kData)[lane] = 0u;
    __syncthreads();

    if constexpr (kBits == 4) {
      // Pack nibbles in the page order of s4kv.h: lane writes its 16-byte block.
      {
        const int t = lane & 15, g = lane >> 4;
        uint32_t dw[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint32_t w = 0;
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            const int d = 32 * m + 8 * g + 2 * (kk & 3) + (kk >> 2);
            w |= static_cast<uint32_t>(kc[t][d]) << (4 * kk);
          }
          dw[m] = w;
        }
        reinterpret_cast<uint4*>(chunk + kOffKCodes)[lane] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
      }
      {
        const int r = lane & 15, g = lane >> 4;
        uint32_t dw[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uint32_t w = 0;
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            const int t = 4 * g + 2 * (kk & 1) + (kk >> 2);
            const int d = 16 * (2 * m + ((kk & 3) >> 1)) + r;
            w |= static_cast<uint32_t>(vc[t][d]) << (4 * kk);
          }
          dw[m] = w;
        }
        reinterpret_cast<uint4*>(chunk + kOffVCodes)[lane] = make_uint4(dw[0], dw[1], dw[2], dw[3]);
      }
    } else {
      // 2-bit codes in the page order of s4kv.h: lane l writes 8 bytes of
      // each code block. K: lane 16g + t holds token t; dword dd carries
      // operands m = 2dd, 2dd + 1, element i (channel 32m + 8g + i) at bit
      // 8 (m & 1) + 2 (i >> 1) + 16 (i & 1).
      {
        const int t = lane & 15, g = lane >> 4;
        uint32_t dw[2];
#pragma unroll
        for (int dd = 0; dd < 2; ++dd) {
          uint32_t w = 0;
#pragma unroll
          for (int mm = 0; mm < 2; ++mm)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int m = 2 * dd + mm;
              w |= static_cast<uint32_t>(kc[t][32 * m + 8 * g + i]) << (8 * mm + 2 * (i >> 1) + 16 * (i & 1));
            }
          dw[dd] = w;
        }
        reinterpret_cast<uint2*>(chunk + C::kK)[lane] = make_uint2(dw[0], dw[1]);
      }
      // V: lane 16g + r holds channel 16 u + r of tokens 4g .. 4g+3 for the
      // 8 tiles u; dword dd carries tiles u = 4dd + sub, token 4g + k at bit
      // 4 sub + 2 (k >> 1) + 16 (k & 1).
      {
        const int r = lane & 15, g = lane >> 4;
        uint32_t dw[2];
#pragma unroll
        for (int dd = 0; dd < 2; ++dd) {
          uint32_t w = 0;
#pragma unroll
          for (int sub = 0; sub < 4; ++sub)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
              w |= static_cast<uint32_t>(vc[4 * g + kk][16 * (4 * dd + sub) + r])
                   << (4 * sub + 2 * (kk >> 1) + 16 * (kk & 1));
          dw[dd] = w;
        }
        reinterpret_cast<uint2*>(chunk + C::kV)[lane] = make_uint2(dw[0], dw[1]);
      }
    }
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
