// Dense paged caches: fp16 (the control path of the int4 cache) and FP8 E4M3
// with per-KV-head scales. Append and decode for both.
//
// The int4 cache replaces an fp16 paged cache. The fp16 path keeps K and V in
// fp16 pages of the same 16 tokens and runs the same decode attention, so the
// two can be timed on one harness. The pages are why the comparison matters:
// the S4 KV product page ("FAQ", the question on inference latency) says the
// int4 backend gives up some decode latency for density at long contexts, and
// the KV-quantization guide on adechristanto.de (section on separating
// weights, running state and reserved memory) notes that a smaller KV element
// halves the payload term, not necessarily the latency.
//
// The FP8 path is the quantized cache that guide discusses most (sections on
// attention arithmetic in the quantized domain and on default or calibrated
// scales): each K and V element is one OCP E4M3 byte, value = code value x the
// KV head's fp32 scale, one scale for K and one for V per KV head.
//
// fp16 pool: fp16 [num_pages][Hkv][4096]. A (page, KV head) chunk holds the K
// block [16 tokens][128 channels], then the V block transposed, [128
// channels][16 tokens], so both matrix-core operands are contiguous 16- and
// 8-byte reads.
//
// FP8 pool: uint8 [num_pages][Hkv][4096], each chunk four 1024-byte blocks in
// matrix-core operand order. Byte 1024 j + 16 L + i belongs to lane L = 16 g +
// c of the decode wave:
//   j = 0, 1: K[token c][channel 32 (2j + i/8) + 8g + i%8]
//   j = 2, 3: V[token 4g + i%4][channel 16 (4(j-2) + i/4) + c]
// A page stage is then four ds_read_b128 at lane-contiguous addresses (no LDS
// bank conflicts), and the bytes a lane reads are exactly the ones its own
// DMA brought in.
//
// Both pools: a sequence's last page may be partial; only its first ctx - 16 *
// (pages - 1) token slots are defined, and the kernel never lets the others
// reach an arithmetic result.
//
// Decode: the persistent split of the int4 path (a flat unit list over
// (b, h, page), W equal contiguous ranges, partial results merged by the shared
// merge kernel), whole pages per stage of an LDS DMA ring (each format sets
// its stage count and pages per stage; 8 waves per CU). The DMA loads are
// non-temporal. A single stage, refilled as soon as the wave has read it into
// registers, measured fastest for both formats: more bytes in flight per wave
// only queue longer.
//  * logits: S^T[token][col] = sum_d K[token][d] q[d][col] on
//    v_mfma_f32_16x16x32_f16, 4 per page; fp16 x fp16 products are exact in
//    the fp32 sums, and E4M3 values convert to fp16 exactly.
//  * output: O^T[d][col] += sum_token V^T[d][token] p[token][col] on
//    v_mfma_f32_16x16x16_f16, 8 per page. The logits' D layout (lane group g
//    holds tokens 4g..4g+3 of its column) is this product's B layout, so the
//    probabilities need no exchange. p enters as an fp16 (hi, lo) pair: for
//    G <= 8, columns c and c + 8 carry one head's hi and lo parts; for G > 8
//    each tile takes two products.
//  * FP8 scales: the K scale folds into the logit scale, the V scale
//    multiplies the partial output once per (sequence, head) segment.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include "internal.h"

namespace s4kv {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -INFINITY;
constexpr float kLog2e = 1.4426950408889634f;
// The reference max of a column moves only when a logit passes it by more
// than this (log2 units); probabilities stay below 2^8, far inside fp16.
constexpr float kLazyRescale = 8.0f;
constexpr int kSlotStride = kHeadDim + 4;  // the shared partial-slot row

__device__ inline f4 mfma32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline f4 mfma16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ inline uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline float bitsf(uint32_t v) { return __builtin_bit_cast(float, v); }
// sum / max over the four 16-lane rows (lanes l ^ 16 and l ^ 32)
__device__ inline float rows_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
  v = bitsf(r[0]) + bitsf(r[1]);
  auto t = __builtin_amdgcn_permlane32_swap(fbits(v), fbits(v), false, false);
  return bitsf(t[0]) + bitsf(t[1]);
}
__device__ inline float rows_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
  v = fmaxf(bitsf(r[0]), bitsf(r[1]));
  auto t = __builtin_amdgcn_permlane32_swap(fbits(v), fbits(v), false, false);
  return fmaxf(bitsf(t[0]), bitsf(t[1]));
}
// v of lane c ^ 8 (c = lane % 16): DPP row rotation by 8
__device__ inline float xor8(float v) {
  return bitsf(static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(fbits(v)), 0x128, 0xF, 0xF, true)));
}

// Every cache byte is read once: the loads carry the non-temporal policy (nt),
// which streams them past the caches; on MI355X a pure read of 4 KB chunks
// runs at about 6.8-7.0 TB/s this way against about 6.0 TB/s without it.
constexpr int kNonTemporal = 2;
__device__ inline void dma16(const uint8_t* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                   (__attribute__((address_space(3))) void*)(lds_base), 16, 0,
                                   kNonTemporal);
}
// s_waitcnt with only vmcnt constrained (gfx9 encoding)
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Wait until the oldest page in flight has landed, when `ahead` later pages
// (Per DMA operations each) may stay outstanding.
template <int Per, int MaxAhead>
__device__ inline void wait_pages_after(int ahead) {
  if constexpr (MaxAhead > 0) {
    if (ahead >= MaxAhead) {
      wait_vmcnt<Per * MaxAhead>();
      return;
    }
    wait_pages_after<Per, MaxAhead - 1>(ahead);
  } else {
    wait_vmcnt<0>();
  }
}
__device__ inline void compiler_fence() { __asm__ __volatile__("" ::: "memory"); }

// ---- page formats ----
// read(): one page of a stage into registers (asm block with its own
// lgkmcnt(0): the caller's vmcnt wait is the only guard the DMA needs).
// keys() / values(): the matrix-core operands of lane (c, g):
//   km[m] = K[token c][32m + 8g .. +7]; vt[t] = V[tokens 4g .. 4g+3][16t + c].

struct F16Pages {
  static constexpr int kChunk = kF16ChunkHalves * 2;  // 8192
  static constexpr int kStages = 1;
  static constexpr int kPagesPerStage = 1;
  static constexpr int kWavesPerSimd = 2;
  static constexpr bool kScaled = false;
  struct Stage {
    u4 k[4];  // K[token c][32m + 8g .. +7], m = 0..3
    u2 v[8];  // V^T[16t + c][4g .. 4g+3], t = 0..7
  };
  __device__ static void read(uint32_t base, int lane, Stage& r) {
    const int c = lane & 15, g = lane >> 4;
    const uint32_t a_k = base + 256 * c + 16 * g;
    const uint32_t a_v = base + 4096 + 32 * c + 8 * g;
    __asm__ __volatile__(
        "ds_read_b128 %0, %12\n\t"
        "ds_read_b128 %1, %12 offset:64\n\t"
        "ds_read_b128 %2, %12 offset:128\n\t"
        "ds_read_b128 %3, %12 offset:192\n\t"
        "ds_read_b64 %4, %13\n\t"
        "ds_read_b64 %5, %13 offset:512\n\t"
        "ds_read_b64 %6, %13 offset:1024\n\t"
        "ds_read_b64 %7, %13 offset:1536\n\t"
        "ds_read_b64 %8, %13 offset:2048\n\t"
        "ds_read_b64 %9, %13 offset:2560\n\t"
        "ds_read_b64 %10, %13 offset:3072\n\t"
        "ds_read_b64 %11, %13 offset:3584\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.k[0]), "=&v"(r.k[1]), "=&v"(r.k[2]), "=&v"(r.k[3]), "=&v"(r.v[0]), "=&v"(r.v[1]),
          "=&v"(r.v[2]), "=&v"(r.v[3]), "=&v"(r.v[4]), "=&v"(r.v[5]), "=&v"(r.v[6]), "=&v"(r.v[7])
        : "v"(a_k), "v"(a_v)
        : "memory");
  }
  __device__ static void keys(const Stage& r, h8 km[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) km[m] = __builtin_bit_cast(h8, r.k[m]);
  }
  __device__ static void values(const Stage& r, h4 vt[8]) {
#pragma unroll
    for (int t = 0; t < 8; ++t) vt[t] = __builtin_bit_cast(h4, r.v[t]);
  }
};

// E4M3 byte pairs to fp16 pairs on the gfx950 converter (scale 1: exact)
__device__ inline h2 e4m3_lo(uint32_t w) { return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false); }
__device__ inline h2 e4m3_hi(uint32_t w) { return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true); }

struct F8Pages {
  static constexpr int kChunk = kF8ChunkBytes;  // 4096
  static constexpr int kStages = 1;
  static constexpr int kPagesPerStage = 1;
  static constexpr int kWavesPerSimd = 2;
  static constexpr bool kScaled = true;
  struct Stage {
    u4 b[4];  // the lane's 16 bytes of blocks 0..3
  };
  __device__ static void read(uint32_t base, int lane, Stage& r) {
    const uint32_t a = base + 16 * lane;
    __asm__ __volatile__(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.b[0]), "=&v"(r.b[1]), "=&v"(r.b[2]), "=&v"(r.b[3])
        : "v"(a)
        : "memory");
  }
  // two consecutive pages of a stage
  __device__ static void read2(uint32_t base, int lane, Stage& r, Stage& s) {
    const uint32_t a = base + 16 * lane;
    __asm__ __volatile__(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\t"
        "ds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b128 %4, %8 offset:4096\n\t"
        "ds_read_b128 %5, %8 offset:5120\n\t"
        "ds_read_b128 %6, %8 offset:6144\n\t"
        "ds_read_b128 %7, %8 offset:7168\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r.b[0]), "=&v"(r.b[1]), "=&v"(r.b[2]), "=&v"(r.b[3]), "=&v"(s.b[0]), "=&v"(s.b[1]),
          "=&v"(s.b[2]), "=&v"(s.b[3])
        : "v"(a)
        : "memory");
  }
  __device__ static void keys(const Stage& r, h8 km[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t w0 = r.b[m >> 1][2 * (m & 1)], w1 = r.b[m >> 1][2 * (m & 1) + 1];
      const h2 a = e4m3_lo(w0), b = e4m3_hi(w0), d = e4m3_lo(w1), e = e4m3_hi(w1);
      km[m] = h8{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
    }
  }
  __device__ static void values(const Stage& r, h4 vt[8]) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t w = r.b[2 + (t >> 2)][t & 3];
      const h2 a = e4m3_lo(w), b = e4m3_hi(w);
      vt[t] = h4{a[0], a[1], b[0], b[1]};
    }
  }
};

// pages of a sequence: full pages plus one for a partial page
__device__ inline int pages_of(int ctx, int max_pages) {
  ctx = min(ctx, max_pages * kPage);
  return ctx > 0 ? (ctx + kPage - 1) / kPage : 0;
}
__device__ inline int owner_wave(int64_t u, int64_t U, int W) {
  return static_cast<int>(((u + 1) * W - 1) / U);
}

template <class Fmt, int G>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(Fmt::kWavesPerSimd, Fmt::kWavesPerSimd))) void dense_stream_kernel(
    const __half* __restrict__ q, const uint8_t* __restrict__ pages,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens,
    int32_t* __restrict__ total_units, int2* __restrict__ seg_waves, int32_t B, int32_t max_pages,
    int32_t hkv, float sm_scale, const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    float* __restrict__ slots) {
  constexpr bool kSplitCols = (G <= 8);  // columns c and c + 8: hi / lo parts of one head
  constexpr int kChunk = Fmt::kChunk;
  constexpr int kStages = Fmt::kStages;
  constexpr int kPer = Fmt::kPagesPerStage;  // pages of one (b, h) per ring stage
  static_assert(kPer == 1 || kPer == 2, "one or two pages per stage");
  constexpr int kDmaPerStage = kPer * kChunk / 1024;
  const int w = blockIdx.x, W = gridDim.x;
  const int lane = threadIdx.x;
  const int c = lane & 15, g = lane >> 4;
  const int hq = hkv * G;

  // ---- unit plan: units(b) = pages of b; (b, h) pairs b-major; W equal ranges ----
  int64_t U;
  {
    int local = 0;
    for (int b = lane; b < B; b += 64) local += pages_of(ctx_lens[b], max_pages);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
    U = (int64_t)hkv * __builtin_amdgcn_readfirstlane(local);
  }
  // Unit indices fit in int32 (the host checks B * Hkv * (max_pages + 1)): the
  // cursors count in 32 bits, so every range check is one scalar compare.
  const int32_t u0 = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((int64_t)w * U / W));
  const int32_t u1 = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((int64_t)(w + 1) * U / W));
  if (w == 0 && lane == 0) total_units[0] = static_cast<int32_t>(U);
  if (u0 >= u1) return;
  int b0 = -1;
  int32_t s0 = 0;  // first unit of sequence b0
  {
    int64_t carry = 0;
    for (int k = 0; k < (B + 63) / 64 && b0 < 0; ++k) {
      const int b = 64 * k + lane;
      const int n = (b < B) ? pages_of(ctx_lens[b], max_pages) : 0;
      int incl = n;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      const int64_t start_b = (int64_t)hkv * (carry + incl - n);
      const uint64_t past = __ballot(b < B && start_b + (int64_t)hkv * n > u0);
      if (past) {
        const int lf = __builtin_ctzll(past);
        b0 = 64 * k + lf;
        s0 = static_cast<int32_t>((int64_t)hkv * (carry + __builtin_amdgcn_readfirstlane(__shfl(incl - n, lf))));
      }
      carry += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
    }
  }
  b0 = __builtin_amdgcn_readfirstlane(b0);

  // Column roles: c = 8*part + hh (G <= 8; part 0 / 1 = hi / lo of p) or c = hh.
  // Columns hh >= G repeat head hh % G so everything they carry stays finite.
  const int hh = kSplitCols ? (c & 7) : c;
  const int head = hh % G;
  const bool lo_col = kSplitCols && c >= 8;
  const float l2s_base = sm_scale * kLog2e;  // logits in log2 units
  const int64_t page_stride = (int64_t)hkv * kChunk;

  struct Cursor {
    int32_t u;   // flat index of the next unit
    int b, h;    // sequence, KV head
    int unit;    // page inside (b, h)
    int npages;  // pages of b
    int last_n;  // tokens in the last page of b
  };
  // cursor fields are wave-uniform; readfirstlane keeps them (and the loads
  // they address) on the scalar unit
  auto seq_info = [&](int b, Cursor& cu) {
    const int ctx = min(ctx_lens[__builtin_amdgcn_readfirstlane(b)], max_pages * kPage);
    cu.npages = ctx > 0 ? (ctx + kPage - 1) / kPage : 0;
    cu.last_n = ctx > 0 ? ctx - kPage * (cu.npages - 1) : 0;
  };
  Cursor start;
  start.u = u0;
  start.b = b0;
  seq_info(b0, start);
  start.h = (u0 - s0) / start.npages;
  start.unit = (u0 - s0) % start.npages;
  auto advance = [&](Cursor& cu) {
    ++cu.u;
    if (++cu.unit >= cu.npages && cu.u < u1) {
      cu.unit = 0;
      if (++cu.h == hkv) {
        cu.h = 0;
        do { ++cu.b; seq_info(cu.b, cu); } while (cu.npages == 0);
      }
    }
  };

  // ---- DMA ring: kPer pages of one (b, h) per stage ----
  // With two pages per stage, a stage whose segment has one page left holds
  // that page twice (the second copy comes from L2 and is fully masked), so
  // every stage is the same number of DMA operations.
  __shared__ __align__(16) uint8_t stage_s[kStages][kPer * kChunk];
  Cursor prod = start;
  int issued = 0, consumed = 0;
  // block ids of the pages at the producer cursor, loaded one stage ahead
  int nid = 0, nid2 = 0;
  auto prefetch_id = [&]() {
    if (prod.u < u1) {
      const int64_t row = (int64_t)__builtin_amdgcn_readfirstlane(prod.b) * max_pages;
      const int un = __builtin_amdgcn_readfirstlane(prod.unit);
      nid = block_table[row + un];
      if constexpr (kPer == 2) nid2 = (un + 1 < prod.npages) ? block_table[row + un + 1] : nid;
    }
  };
  // the second page of a stage exists when the cursor, moved past the first,
  // is still inside the range and the same (b, h)
  auto has_second = [&](const Cursor& cu) { return cu.u < u1 && cu.unit != 0; };
  auto produce = [&]() {
    if (prod.u >= u1) return;
    const int64_t head_off = (int64_t)prod.h * kChunk + 16 * lane;
    const uint8_t* ch = pages + nid * page_stride + head_off;
    const uint8_t* ch2 = ch;
    advance(prod);
    if constexpr (kPer == 2) {
      if (has_second(prod)) {
        ch2 = pages + nid2 * page_stride + head_off;
        advance(prod);
      }
    }
    uint8_t* st = stage_s[issued % kStages];
#pragma unroll
    for (int i = 0; i < kChunk / 1024; ++i) dma16(ch + 1024 * i, st + 1024 * i);
    if constexpr (kPer == 2) {
#pragma unroll
      for (int i = 0; i < kChunk / 1024; ++i) dma16(ch2 + 1024 * i, st + kChunk + 1024 * i);
    }
    ++issued;
    prefetch_id();
  };

  // ---- per-(b, h) state, per column ----
  h8 qv[4];  // query of the column's head: element i of product m is channel 32m+8g+i
  float m_run = kNegInf, l_part = 0.f;
  float l2s = l2s_base;
  f4 o[8];
  int cur_b = -1, cur_h = 0;

  auto begin_segment = [&](const Cursor& cu) {
    cur_b = cu.b;
    cur_h = cu.h;
    const int32_t first = cu.u - cu.unit;
    if (first >= u0 && lane == 0)
      seg_waves[(int64_t)cu.b * hkv + cu.h] =
          make_int2(owner_wave(first, U, W), owner_wave(first + cu.npages - 1, U, W));
    const uint8_t* qr = reinterpret_cast<const uint8_t*>(q + ((int64_t)cu.b * hq + cu.h * G + head) * kHeadDim);
#pragma unroll
    for (int m = 0; m < 4; ++m) qv[m] = __builtin_bit_cast(h8, *reinterpret_cast<const u4*>(qr + 2 * (32 * m + 8 * g)));
    if constexpr (Fmt::kScaled) l2s = l2s_base * k_scale[__builtin_amdgcn_readfirstlane(cu.h)];
    m_run = kNegInf;
    l_part = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = f4{0.f, 0.f, 0.f, 0.f};
  };
  auto end_segment = [&]() {
    const float l = rows_sum(l_part);
    if constexpr (kSplitCols) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[t][i] += xor8(o[t][i]);
    }
    if constexpr (Fmt::kScaled) {
      const float vs = v_scale[__builtin_amdgcn_readfirstlane(cur_h)];
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= vs;
    }
    if (c < G) {
      const int64_t slot = (int64_t)cur_b * hkv + cur_h + w;
      float* dst = slots + (slot * G + c) * kSlotStride;
#pragma unroll
      for (int t = 0; t < 8; ++t) *reinterpret_cast<f4*>(dst + 16 * t + 4 * g) = o[t];
      if (g == 0) { dst[kHeadDim] = m_run; dst[kHeadDim + 1] = l; }
    }
  };

  auto lds_addr = [&](const uint8_t* p) -> uint32_t {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)(p)));
  };
  // n_valid[pg]: defined tokens of page pg of the stage (16, fewer on a
  // sequence's last page, 0 for the repeated copy of a lone page)
  auto process_stage = [&](const uint8_t* st, const int (&n_valid)[kPer]) {
    typename Fmt::Stage r[kPer];
    if constexpr (kPer == 2) Fmt::read2(lds_addr(st), lane, r[0], r[1]);
    else Fmt::read(lds_addr(st), lane, r[0]);
    // the stage is in registers: refill it at once
    compiler_fence();
    produce();
    compiler_fence();
    float lg[kPer][4];
#pragma unroll
    for (int pg = 0; pg < kPer; ++pg) {
      h8 km[4];
      Fmt::keys(r[pg], km);
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) acc = mfma32(km[m], qv[m], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) lg[pg][i] = (4 * g + i < n_valid[pg]) ? acc[i] * l2s : kNegInf;
    }
    float mx = fmaxf(fmaxf(lg[0][0], lg[0][1]), fmaxf(lg[0][2], lg[0][3]));
#pragma unroll
    for (int pg = 1; pg < kPer; ++pg)
      mx = fmaxf(mx, fmaxf(fmaxf(lg[pg][0], lg[pg][1]), fmaxf(lg[pg][2], lg[pg][3])));
    const float mb = rows_max(mx);
    const bool up = mb > m_run + kLazyRescale;
    if (__any(up)) {
      const float mnew = up ? mb : m_run;
      const float alpha = (mnew == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - mnew);
      l_part *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= alpha;
      m_run = mnew;
    }
    const float ms = (m_run == kNegInf) ? 0.f : m_run;
#pragma unroll
    for (int pg = 0; pg < kPer; ++pg) {
      h4 bh, bl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(lg[pg][i] - ms);
        l_part += p;
        const _Float16 ph = static_cast<_Float16>(p);
        bh[i] = ph;
        bl[i] = static_cast<_Float16>(p - static_cast<float>(ph));
      }
      h4 vt[8];
      Fmt::values(r[pg], vt);
      if (n_valid[pg] < kPage) {
        // undefined slots of a partial page: their probabilities are 0, and
        // their values must not be NaN or Inf either
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * g + i >= n_valid[pg]) vt[t][i] = static_cast<_Float16>(0.f);
      }
      if constexpr (kSplitCols) {
        const h4 b = lo_col ? bl : bh;
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] = mfma16(vt[t], b, o[t]);
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          o[t] = mfma16(vt[t], bh, o[t]);
          o[t] = mfma16(vt[t], bl, o[t]);
        }
      }
    }
  };

  // ---- main stream ----
  // kStages stages are issued ahead; loads complete in issue order, so "at
  // most kDmaPerStage x (stages issued after this one)" outstanding
  // vector-memory operations means this stage has landed. Other outstanding
  // operations (query loads, partial stores) can only make the wait stricter.
  prefetch_id();
#pragma unroll
  for (int s = 0; s < kStages; ++s) produce();
  Cursor cons = start;
  while (cons.u < u1) {
    begin_segment(cons);
    do {
      // the consumer walks the same stage boundaries as the producer
      int n_valid[kPer];
      n_valid[0] = (cons.unit == cons.npages - 1) ? cons.last_n : kPage;
      advance(cons);
      if constexpr (kPer == 2) {
        n_valid[1] = 0;
        if (has_second(cons)) {
          n_valid[1] = (cons.unit == cons.npages - 1) ? cons.last_n : kPage;
          advance(cons);
        }
      }
      wait_pages_after<kDmaPerStage, kStages - 1>(issued - consumed - 1);
      compiler_fence();
      process_stage(stage_s[consumed % kStages], n_valid);
      compiler_fence();
      ++consumed;
    } while (cons.u < u1 && cons.b == cur_b && cons.h == cur_h);
    end_segment();
  }
}

// One work-group per (page slot of the append, KV head, sequence); lane l
// owns channels 2l and 2l + 1.
__global__ __launch_bounds__(64) void fp16_append_kernel(
    const __half* __restrict__ k, const __half* __restrict__ v, const int32_t* __restrict__ cu_new,
    const int32_t* __restrict__ slot, const int32_t* __restrict__ block_table, int32_t max_pages,
    __half* __restrict__ pages, int32_t hkv) {
  const int x = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int start = slot[b];
  const int64_t row0 = cu_new[b];
  const int n = cu_new[b + 1] - cu_new[b];
  if (n <= 0) return;
  const int end = start + n;
  const int p = start / kPage + x;
  if (p > (end - 1) / kPage) return;
  __half* chunk = pages + ((int64_t)block_table[(int64_t)b * max_pages + p] * hkv + h) * kF16ChunkHalves;
  const int t0 = max(start, p * kPage), t1 = min(end, (p + 1) * kPage);
  for (int t = t0; t < t1; ++t) {
    const int64_t row = ((row0 + (t - start)) * hkv + h) * kHeadDim;
    const int ts = t % kPage;
    reinterpret_cast<__half2*>(chunk + ts * kHeadDim)[lane] = reinterpret_cast<const __half2*>(k + row)[lane];
    const __half2 vv = reinterpret_cast<const __half2*>(v + row)[lane];
    chunk[kPage * kHeadDim + (2 * lane) * kPage + ts] = __low2half(vv);
    chunk[kPage * kHeadDim + (2 * lane + 1) * kPage + ts] = __high2half(vv);
  }
}

// OCP E4M3 code of an fp32 value: round to nearest, ties to even, magnitudes
// of 448 and above saturate to 448 (code 0x7E), the sign is kept (also for a
// zero result). Written from the format: 1 sign, 4 exponent bits of bias 7, 3
// mantissa bits; below 2^-6 the codes are the multiples of 2^-9.
__device__ inline uint32_t e4m3_code(float y) {
  const uint32_t sign = (fbits(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t mag;
  if (!(a < 448.0f)) {
    mag = 0x7Eu;
  } else if (a < 0x1p-6f) {
    mag = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));  // exact scaling, then RNE
  } else {
    // fp32 bits >> 20 = (biased exponent << 3) | top 3 mantissa bits; adding
    // 2^19 - 1 plus the kept LSB rounds the dropped 20 bits to nearest-even,
    // a carry moving into the exponent. Rebias 127 -> 7.
    const uint32_t ab = fbits(a);
    mag = min(((ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20) - (120u << 3), 0x7Eu);
  }
  return sign | mag;
}

// FP8 append: one work-group per (page slot of the append, KV head,
// sequence); lane l owns channels 2l and 2l + 1. Codes go to the operand-order
// layout described at the top of this file.
__global__ __launch_bounds__(64) void fp8_append_kernel(
    const __half* __restrict__ k, const __half* __restrict__ v, const int32_t* __restrict__ cu_new,
    const int32_t* __restrict__ slot, const int32_t* __restrict__ block_table, int32_t max_pages,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, uint8_t* __restrict__ pages,
    int32_t hkv) {
  const int x = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int start = slot[b];
  const int64_t row0 = cu_new[b];
  const int n = cu_new[b + 1] - cu_new[b];
  if (n <= 0) return;
  const int end = start + n;
  const int p = start / kPage + x;
  if (p > (end - 1) / kPage) return;
  uint8_t* chunk = pages + ((int64_t)block_table[(int64_t)b * max_pages + p] * hkv + h) * kF8ChunkBytes;
  const float ks = k_scale[h], vs = v_scale[h];
  // K channel 2l: m = l / 16, g = (l / 4) % 4, byte (2l) % 8 of half m % 2
  const int m = lane >> 4;
  const int k_off = 1024 * (m >> 1) + 16 * 16 * ((lane >> 2) & 3) + 8 * (m & 1) + ((2 * lane) & 7);
  // V channels 2l, 2l + 1: t = l / 8, c = (2l) % 16 (+1)
  const int t = lane >> 3;
  const int v_off = 1024 * (2 + (t >> 2)) + 16 * ((2 * lane) & 15) + 4 * (t & 3);
  const int t0 = max(start, p * kPage), t1 = min(end, (p + 1) * kPage);
  for (int tok = t0; tok < t1; ++tok) {
    const int64_t row = ((row0 + (tok - start)) * hkv + h) * kHeadDim;
    const int ts = tok % kPage;
    const __half2 kk = reinterpret_cast<const __half2*>(k + row)[lane];
    const __half2 vv = reinterpret_cast<const __half2*>(v + row)[lane];
    const uint32_t k0 = e4m3_code(__low2float(kk) / ks), k1 = e4m3_code(__high2float(kk) / ks);
    *reinterpret_cast<uint16_t*>(chunk + k_off + 16 * ts) = static_cast<uint16_t>(k0 | (k1 << 8));
    const int vo = v_off + 16 * 16 * (ts >> 2) + (ts & 3);
    chunk[vo] = static_cast<uint8_t>(e4m3_code(__low2float(vv) / vs));
    chunk[vo + 16] = static_cast<uint8_t>(e4m3_code(__high2float(vv) / vs));
  }
}

template <class Fmt, int G>
hipError_t launch_dense_g(const s4kv_shape& s, int W, const void* q, const void* pages,
                          const int32_t* block_table, const int32_t* ctx_lens, const SplitWorkspace& ws,
                          float sm_scale, const float* k_scale, const float* v_scale, hipStream_t stream) {
  hipLaunchKernelGGL((dense_stream_kernel<Fmt, G>), dim3(W), dim3(64), 0, stream,
                     static_cast<const __half*>(q), static_cast<const uint8_t*>(pages), block_table,
                     ctx_lens, ws.total_units, reinterpret_cast<int2*>(ws.seg_waves), s.num_seqs,
                     s.max_pages_per_seq, s.num_kv_heads, sm_scale, k_scale, v_scale, ws.slots);
  return hipGetLastError();
}

template <class Fmt>
hipError_t launch_dense_decode(const s4kv_shape& s, const void* q, const void* pages,
                               const int32_t* block_table, const int32_t* ctx_lens, int32_t max_ctx,
                               float sm_scale, const float* k_scale, const float* v_scale, void* out,
                               void* workspace, hipStream_t stream) {
  const SplitWorkspace ws = split_workspace(s, workspace);
  // resident_waves() is two per SIMD
  const int W = min(resident_waves() / 2 * Fmt::kWavesPerSimd, kMaxWaves);
  const int G = s.num_q_heads / s.num_kv_heads;
  hipError_t e = hipSuccess;
  switch (G) {
#define S4KV_DENSE_CASE(g)                                                                        \
  case g:                                                                                         \
    e = launch_dense_g<Fmt, g>(s, W, q, pages, block_table, ctx_lens, ws, sm_scale, k_scale, v_scale, \
                               stream);                                                           \
    break;
    S4KV_DENSE_CASE(1) S4KV_DENSE_CASE(2) S4KV_DENSE_CASE(3) S4KV_DENSE_CASE(4) S4KV_DENSE_CASE(5)
    S4KV_DENSE_CASE(6) S4KV_DENSE_CASE(7) S4KV_DENSE_CASE(8) S4KV_DENSE_CASE(9) S4KV_DENSE_CASE(10)
    S4KV_DENSE_CASE(11) S4KV_DENSE_CASE(12) S4KV_DENSE_CASE(13) S4KV_DENSE_CASE(14)
    S4KV_DENSE_CASE(15) S4KV_DENSE_CASE(16)
#undef S4KV_DENSE_CASE
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_split_merge(s, W, max_ctx, ws, ctx_lens, out, stream);
}

// pages touched by n tokens starting anywhere inside a page: floor((n+14)/16)+1
inline int append_page_slots(int32_t max_new) { return (max_new + 14) / kPage + 1; }

}  // namespace

hipError_t launch_fp16_append(const s4kv_shape& s, const void* k, const void* v,
                              const int32_t* cu_new, const int32_t* slot, int32_t max_new,
                              const int32_t* block_table, void* pages, hipStream_t stream) {
  hipLaunchKernelGGL(fp16_append_kernel, dim3(append_page_slots(max_new), s.num_kv_heads, s.num_seqs),
                     dim3(64), 0, stream, static_cast<const __half*>(k), static_cast<const __half*>(v),
                     cu_new, slot, block_table, s.max_pages_per_seq, static_cast<__half*>(pages),
                     s.num_kv_heads);
  return hipGetLastError();
}

hipError_t launch_fp16_decode(const s4kv_shape& s, const void* q, const void* pages,
                              const int32_t* block_table, const int32_t* ctx_lens, int32_t max_ctx,
                              float sm_scale, void* out, void* workspace, hipStream_t stream) {
  return launch_dense_decode<F16Pages>(s, q, pages, block_table, ctx_lens, max_ctx, sm_scale, nullptr,
                                       nullptr, out, workspace, stream);
}

hipError_t launch_fp8_append(const s4kv_shape& s, const void* k, const void* v, const int32_t* cu_new,
                             const int32_t* slot, int32_t max_new, const int32_t* block_table,
                             const float* k_scale, const float* v_scale, void* pages, hipStream_t stream) {
  hipLaunchKernelGGL(fp8_append_kernel, dim3(append_page_slots(max_new), s.num_kv_heads, s.num_seqs),
                     dim3(64), 0, stream, static_cast<const __half*>(k), static_cast<const __half*>(v),
                     cu_new, slot, block_table, s.max_pages_per_seq, k_scale, v_scale,
                     static_cast<uint8_t*>(pages), s.num_kv_heads);
  return hipGetLastError();
}

hipError_t launch_fp8_decode(const s4kv_shape& s, const void* q, const void* pages,
                             const int32_t* block_table, const int32_t* ctx_lens, int32_t max_ctx,
                             float sm_scale, const float* k_scale, const float* v_scale, void* out,
                             void* workspace, hipStream_t stream) {
  return launch_dense_decode<F8Pages>(s, q, pages, block_table, ctx_lens, max_ctx, sm_scale, k_scale,
                                      v_scale, out, workspace, stream);
}

}  // namespace s4kv
