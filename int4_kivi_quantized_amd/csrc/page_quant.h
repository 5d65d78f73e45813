// Quantization of one full page (16 tokens x 128 channels of one KV head)
// into the page format of s4kv.h, by one 64-lane wave. Shared by the append
// kernel and by the decode call that appends one token per sequence.
//
// Method: S4 KV product page ("Funktionsweise" step 1): asymmetric codes,
// KEY grouped per channel over the page's 16 tokens, VALUE per token over
// its 128 channels; zero = group minimum, scale = (max - min) / qmax rounded
// to fp16, codes from the stored fp16 scale and zero. The 2-bit instance is
// the KIVI variant the KV-cache explainer cites (analyticslegends.ai,
// "Quellen", entry 17): qmax 3 instead of 15.
//
// Rounding is fixed so that codes are reproducible bit for bit: IEEE fp32
// subtract and correctly rounded divide, round half to even, clamp to
// [0, qmax]; no contraction into fused multiply-adds.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "internal.h"

namespace s4kv {

// Code width: page geometry and the largest code.
template <int kBits>
struct Codes;
template <>
struct Codes<4> {
  static constexpr float kQmax = 15.0f;
  static constexpr int kStride = kChunkStride, kData = kChunkBytes;
  static constexpr int kK = kOffKCodes, kV = kOffVCodes, kKs = kOffKScale, kKz = kOffKZero,
                       kVs = kOffVScale, kVz = kOffVZero;
  using Block = uint4;  // a lane's share of a code block (16 bytes at 16 * lane)
};
template <>
struct Codes<2> {
  static constexpr float kQmax = 3.0f;
  static constexpr int kStride = kK2ChunkStride, kData = kK2ChunkBytes;
  static constexpr int kK = kOff2KCodes, kV = kOff2VCodes, kKs = kOff2KScale, kKz = kOff2KZero,
                       kVs = kOff2VScale, kVz = kOff2VZero;
  using Block = uint2;  // 8 bytes at 8 * lane
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
#pragma clang fp contract(off)
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
#pragma clang fp contract(off)
  if (g.sf == 0.0f) return 0u;
  float t = rintf((x - g.zf) / g.sf);
  t = fminf(fmaxf(t, 0.0f), Codes<kBits>::kQmax);
  return static_cast<uint32_t>(t);
}

// A lane's share of a quantized page: its blocks of the two code regions,
// the K scale / zero of channels 2 * lane and 2 * lane + 1, and (for lanes
// with lane % 4 == 0) the V scale / zero of token lane / 4.
template <int kBits>
struct PageShare {
  typename Codes<kBits>::Block kcode, vcode;
  __half2 ks, kz;
  __half vs, vz;
};

// Quantize the page whose token t has K row krow(t) and V row vrow(t)
// (128 fp16 each). kc / vc: 16 x 128 bytes of LDS scratch for the codes.
// kmeta(out) / vmeta(out) are called as soon as the K / V scales and zeros
// are known, so a caller can store them while the rest is computed. Every
// lane of the wave must call it (it synchronizes the work-group, which is
// this one wave).
template <int kBits, class RowK, class RowV, class KMeta, class VMeta>
__device__ inline void quantize_page(RowK krow, RowV vrow, int lane, uint8_t (*kc)[kHeadDim],
                                     uint8_t (*vc)[kHeadDim], PageShare<kBits>& out, KMeta kmeta,
                                     VMeta vmeta) {
  // K: lane owns channels 2*lane, 2*lane+1; groups run over the 16 tokens.
  float k0[kPage], k1[kPage];
#pragma unroll
  for (int t = 0; t < kPage; ++t) {
    const __half2 v2 = reinterpret_cast<const __half2*>(krow(t))[lane];
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
  out.ks = __halves2half2(g0.s, g1.s);
  out.kz = __halves2half2(g0.z, g1.z);
  kmeta(out);

  // V: lane owns token t = lane/4, channels 32*(lane%4) .. +32; groups run
  // over the token's 128 channels (4 lanes per token).
  const int vt = lane >> 2, vu = lane & 3;
  const __half* vrow_p = vrow(vt) + 32 * vu;
  float vx[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = reinterpret_cast<const uint4*>(vrow_p)[i];
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
  out.vs = gv.s;
  out.vz = gv.z;
  vmeta(out);
  __syncthreads();

  if constexpr (kBits == 4) {
    // Nibbles in the page order of s4kv.h: the lane's 16-byte block of each region.
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
      out.kcode = make_uint4(dw[0], dw[1], dw[2], dw[3]);
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
      out.vcode = make_uint4(dw[0], dw[1], dw[2], dw[3]);
    }
  } else {
    // 2-bit codes in the page order of s4kv.h: lane l's 8 bytes of each code
    // block. K: lane 16g + t holds token t; dword dd carries operands m = 2dd,
    // 2dd + 1, element i (channel 32m + 8g + i) at bit 8 (m & 1) + 2 (i >> 1)
    // + 16 (i & 1).
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
      out.kcode = make_uint2(dw[0], dw[1]);
    }
    // V: lane 16g + r holds channel 16 u + r of tokens 4g .. 4g+3 for the 8
    // tiles u; dword dd carries tiles u = 4dd + sub, token 4g + k at bit
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
      out.vcode = make_uint2(dw[0], dw[1]);
    }
  }
}

// Store a lane's share of a page at chunk (the page's first byte; global or
// LDS pointer): the K scales and zeros, the V scales and zeros (with
// zero_pad also the padding after the data), the codes, or all of them.
template <int kBits, class Ptr>
__device__ inline void store_page_kmeta(Ptr chunk, int lane, const PageShare<kBits>& in) {
  using C = Codes<kBits>;
  reinterpret_cast<__half2*>(chunk + C::kKs)[lane] = in.ks;
  reinterpret_cast<__half2*>(chunk + C::kKz)[lane] = in.kz;
}
template <int kBits, class Ptr>
__device__ inline void store_page_vmeta(Ptr chunk, int lane, const PageShare<kBits>& in, bool zero_pad) {
  using C = Codes<kBits>;
  if ((lane & 3) == 0) {
    reinterpret_cast<__half*>(chunk + C::kVs)[lane >> 2] = in.vs;
    reinterpret_cast<__half*>(chunk + C::kVz)[lane >> 2] = in.vz;
  }
  if (zero_pad && lane < (C::kStride - C::kData) / 4)
    reinterpret_cast<uint32_t*>(chunk + C::kData)[lane] = 0u;
}
template <int kBits, class Ptr>
__device__ inline void store_page_codes(Ptr chunk, int lane, const PageShare<kBits>& in) {
  using Block = typename Codes<kBits>::Block;
  reinterpret_cast<Block*>(chunk + Codes<kBits>::kK)[lane] = in.kcode;
  reinterpret_cast<Block*>(chunk + Codes<kBits>::kV)[lane] = in.vcode;
}
template <int kBits, class Ptr>
__device__ inline void store_page(Ptr chunk, int lane, const PageShare<kBits>& in, bool zero_pad) {
  store_page_codes<kBits>(chunk, lane, in);
  store_page_kmeta<kBits>(chunk, lane, in);
  store_page_vmeta<kBits>(chunk, lane, in, zero_pad);
}

}  // namespace s4kv
