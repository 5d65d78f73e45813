// Split-K paged decode over the int4 KIVI cache on gfx950 matrix cores.
//
// Method: S4 KV product page ("Funktionsweise" step 1): the paged-attention KV
// cache is stored as int4, KEY per channel (scale/zero per channel for each
// 16-token page), VALUE per token (scale/zero per token); the decode step is
// standard attention (header paragraph: head_dim 128, standard attention),
// with the G = Hq/Hkv query heads of a KV head reading the same pages (GQA,
// KV-cache explainer, "Begriffe", entry "Grouped-Query Attention").
//
// Work decomposition (persistent, balanced): the work of one launch is the flat
// list of "units" over (sequence b, KV head h) in order, a unit being one full
// int4 page or the fp16 tail of (b, h). A fixed grid of W one-wave
// work-groups (as many as the GPU keeps resident) splits the list into W equal
// contiguous ranges; every wave derives the per-sequence unit counts and its
// own range from the context lengths. Each wave streams its range through an HBM -> LDS DMA ring
// (one stage in flight while one is computed), pairing consecutive pages of
// the same (b, h), and keeps an online softmax
// (running max in log2 units, running sum, unnormalized output) for the G
// query heads of the current (b, h); each (b, h) its range touches yields a
// partial result in workspace slot (b*Hkv + h) + wave.
// splitk_reduce_kernel merges, for each (b, query head), the partials of the
// consecutive waves whose ranges touched it.
//
// The same stream can first append one token per sequence (the decode step's
// quantize-on-append, S4 KV product page, "Funktionsweise" step 1): the wave
// owning the last unit of a (b, h) stores the token in the tail, or quantizes
// the page it completes, and attends over it from its inputs (kAppend below).
//
// Dense contractions on v_mfma_f32_16x16x32_f16 (D = A x B, 16x32 by 32x16):
//  * logits, transposed: S^T[token][col] = sum_d codeK[token][d] * qs[d][col]
//    with qs = q * sK (the per-channel K scale folded into the query, per page)
//    plus the zero-point term sum_d q[d] * zK[d] (one number per head and page).
//  * output, transposed: O^T[d][col] += sum_slot codeV^T[d][slot] * ps[slot][col]
//    with ps = p * sV (the per-token V scale folded into the probabilities);
//    the 32 K-slots are 4 tokens of page A and 4 of page B per lane group.
//  * column roles: for G <= 8 a column belongs to one (head, page of the pair):
//    its logits operand carries that page's K scale and its output operand
//    only that page's slots, so neither product needs data from another
//    column; for G <= 4 the free columns carry the low fp16 part of the
//    output operand. Each column keeps its own running max; the page halves
//    (and hi / lo parts) are merged once per (sequence, head) segment. For
//    G > 8 a column is a head and spans both pages.
//  * fp16 hi/lo pairs keep ~22 significant bits in qs and ps, so the products
//    add no error beyond fp32 accumulation order.
//  * the 4-bit codes enter the matrix cores as fp16 subnormals: masking a
//    packed dword with 0x000F000F gives two codes as c * 2^-24, with 0x00F000F0
//    two more as c * 2^-20. Those scale factors are folded into the other
//    operand, so unpacking costs one shift and four ANDs per eight codes.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include <mutex>
#include <type_traits>

#include "internal.h"
#include "page_quant.h"

// The decode workspace of s4kv_paged_decode_append_noalloc, for callers that
// cannot allocate: one copy of this array per device, held until the process
// ends. Host code reaches it only through the address hipGetSymbolAddress
// returns for the current device (noalloc_scratch below).
static __device__ __align__(256) uint8_t scratch[S4KV_NOALLOC_SCRATCH_BYTES];

namespace s4kv {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -INFINITY;
// Running max of a column that has seen no token yet: finite, so exp2(x - m)
// needs no special case (a -inf logit still gives 0, and the first finite
// logit, at most ~2^40 in magnitude for fp16 operands, replaces it with a
// rescale factor of exactly 0).
constexpr float kMEmpty = -1.0e30f;
constexpr float kLog2e = 1.4426950408889634f;
// Codes are fed as c * 2^-24 (slots 0,1,4,5) and c * 2^-20 (slots 2,3,6,7);
// the query side carries 2^-4 and 2^-8 on those slots so every product is
// c * q * s * 2^-28, and the output side carries 1 and 1/16 so every product
// is c * p * s * 2^-24.
constexpr float kQkUnscale = 268435456.0f;  // 2^28
constexpr float kPvUnscale = 16777216.0f;   // 2^24

__device__ inline h8 as_h8(u4 v) { return __builtin_bit_cast(h8, v); }

__device__ inline f4 mfma(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Eight K codes of one dword -> the 8 A-operand elements of one logits product.
__device__ inline h8 k_operand(uint32_t w) {
  const uint32_t w8 = w >> 8;
  u4 v;
  v[0] = w & 0x000F000Fu;
  v[1] = w & 0x00F000F0u;
  v[2] = w8 & 0x000F000Fu;
  v[3] = w8 & 0x00F000F0u;
  return as_h8(v);
}

// V operand of tile pair (2m, 2m+1) from dword m of page A (wa) and page B (wb).
__device__ inline void v_operands(uint32_t wa, uint32_t wb, h8& even, h8& odd) {
  const uint32_t a8 = wa >> 8, b8 = wb >> 8;
  u4 e, o;
  e[0] = wa & 0x000F000Fu; e[1] = wa & 0x00F000F0u; e[2] = wb & 0x000F000Fu; e[3] = wb & 0x00F000F0u;
  o[0] = a8 & 0x000F000Fu; o[1] = a8 & 0x00F000F0u; o[2] = b8 & 0x000F000Fu; o[3] = b8 & 0x00F000F0u;
  even = as_h8(e);
  odd = as_h8(o);
}

// 2-bit codes (pages of the 2-bit format): a mask keeps two codes per dword,
// one in each fp16 half; a code at bits 2j..2j+1 of its half (j = 0..3) is
// the fp16 subnormal c * 2^(2j - 24). K operand m comes from dword m / 2 of
// the lane's 8 bytes, shifted by 8 for odd m, and element i sits at j = i / 2:
// the four element pairs carry 2^-24, 2^-22, 2^-20, 2^-18, and the query
// side carries 2^-4, 2^-6, 2^-8, 2^-10 on them (every product c q s 2^-28).
constexpr uint32_t kM2[4] = {0x00030003u, 0x000C000Cu, 0x00300030u, 0x00C000C0u};
__device__ inline h8 k_operand2(uint32_t w, int odd) {
  const uint32_t x = odd ? (w >> 8) : w;
  u4 v;
  v[0] = x & kM2[0];
  v[1] = x & kM2[1];
  v[2] = x & kM2[2];
  v[3] = x & kM2[3];
  return as_h8(v);
}
// V tiles 2m and 2m+1 of a pair: tile u lives in dword u / 4 of each page at
// shift 4 (u % 4); elements 0..3 from page A, 4..7 from page B. The odd tile
// is taken in place (j = 2, 3: 2^-20 and 2^-18 where the even tile has 2^-24
// and 2^-22), so its products carry 2^-20 where the even tile's carry 2^-24
// (PairFmt::kOddTileUnscale undoes that).
__device__ inline void v_operands2(uint32_t wa, uint32_t wb, int m, h8& even, h8& odd) {
  const int sh = 8 * (m & 1);
  const uint32_t ea = wa >> sh, eb = wb >> sh;
  u4 e, o;
  e[0] = ea & kM2[0]; e[1] = ea & kM2[1]; e[2] = eb & kM2[0]; e[3] = eb & kM2[1];
  o[0] = ea & kM2[2]; o[1] = ea & kM2[3]; o[2] = eb & kM2[2]; o[3] = eb & kM2[3];
  even = as_h8(e);
  odd = as_h8(o);
}

__device__ inline u4 ld16(const uint8_t* p) { return *reinterpret_cast<const u4*>(p); }
__device__ inline u2 ld8(const uint8_t* p) { return *reinterpret_cast<const u2*>(p); }

// Operands of a pair by code width (u4: a lane's 16 int4 bytes, u2: its 8
// 2-bit bytes).
__device__ inline h8 k_op(const u4& kc, int m) { return k_operand(kc[m]); }
__device__ inline h8 k_op(const u2& kc, int m) { return k_operand2(kc[m >> 1], m & 1); }
__device__ inline void v_ops(const u4& a, const u4& b, int m, h8& even, h8& odd) {
  v_operands(a[m], b[m], even, odd);
}
__device__ inline void v_ops(const u2& a, const u2& b, int m, h8& even, h8& odd) {
  v_operands2(a[m >> 1], b[m >> 1], m, even, odd);
}

__device__ inline _Float16 h_at(u4 v, int i) { return __builtin_bit_cast(h8, v)[i]; }
__device__ inline _Float16 h_at2(u2 v, int i) {
  return __builtin_bit_cast(h2v, (uint32_t)v[i >> 1])[i & 1];
}

// ---- cross-lane steps on the VALU (no LDS round trip) ----
__device__ inline uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline float bitsf(uint32_t v) { return __builtin_bit_cast(float, v); }
// v from lane l ^ 16 and from lane l ^ 32 combined with v itself (sum / max
// over the four 16-lane rows): permlane16_swap pairs rows 0-1 and 2-3,
// permlane32_swap pairs the two halves of the wave.
__device__ inline float rows_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
  v = bitsf(r[0]) + bitsf(r[1]);
  auto t = __builtin_amdgcn_permlane32_swap(fbits(v), fbits(v), false, false);
  return bitsf(t[0]) + bitsf(t[1]);
}
// max(a, b) in one instruction: fmaxf on values that come from a lane permute
// first quiets each operand (two more instructions), and the compiler turns
// med3(a, b, +inf) back into that. The operands are never NaN here.
__device__ inline float max2(float a, float b) {
  float r;
  __asm__("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ inline float rows_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(fbits(v), fbits(v), false, false);
  v = max2(bitsf(r[0]), bitsf(r[1]));
  auto t = __builtin_amdgcn_permlane32_swap(fbits(v), fbits(v), false, false);
  return max2(bitsf(t[0]), bitsf(t[1]));
}
// DPP row rotations (within rows of 16 lanes); every lane reads a valid
// source, so no "old" value is needed.
constexpr int kDppRowRor4 = 0x124;    // row_ror:4  (lane c <- c-4 mod 16)
constexpr int kDppRowRor8 = 0x128;    // row_ror:8  (lane c <- c^8)
constexpr int kDppRowRor12 = 0x12C;   // row_ror:12 (lane c <- c+4 mod 16)
template <int Ctrl>
__device__ inline float dpp(float v) {
  return bitsf(static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(fbits(v)), Ctrl, 0xF, 0xF, true)));
}
// v of lane c ^ 8 / c ^ 4 (c = lane % 16)
__device__ inline float xor8(float v) { return dpp<kDppRowRor8>(v); }
__device__ inline float xor4(float v, int c) {
  const float up = dpp<kDppRowRor12>(v);   // from c + 4
  const float dn = dpp<kDppRowRor4>(v);    // from c - 4
  return (c & 4) ? dn : up;
}

// qs = qc * s as an fp16 (hi, lo) pair for the 8 elements of one product,
// two elements per packed fp16 instruction: hi = fp16(qc*s) (one rounding of
// the exact product) and lo = fma(qc, s, -hi) (exact product minus hi, one
// rounding), so hi + lo carries about 22 significant bits of qc*s.
__device__ inline void qs_split(h8 qc, u4 s, h8& hi, h8& lo) {
  const h8 sv = as_h8(s);
  hi = qc * sv;
  lo = __builtin_elementwise_fma(qc, sv, -hi);
}

__device__ inline h2v half_pair(h8 v, int k) { return h2v{v[2 * k], v[2 * k + 1]}; }

// Zero-point terms of the logits, sum_d q[d] * zK[d], for both pages of a
// pair in one chain of products: rows 0..7 of A are page A's K zeros and rows
// 8..15 page B's (lane (c, g) supplies row c, its 8 channels of product m), B
// is the plain query of the lane's head. D rows 4g..4g+3 sit in the lanes of
// group g, so lanes 0..31 hold page A's term for their column and lanes
// 32..63 page B's; swapping the two halves gives every lane both. fp16 x fp16
// products are exact in the fp32 accumulation.
__device__ inline void zero_terms(const h8 (&qh)[4], const u4 (&z)[4], float& ta, float& tb) {
  f4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 4; ++m) d = mfma(as_h8(z[m]), qh[m], d);
  // permlane32_swap(x, x): first result = x of lane l % 32 (lower half),
  // second = x of lane 32 + l % 32 (upper half)
  const auto r = __builtin_amdgcn_permlane32_swap(fbits(d[0]), fbits(d[0]), false, false);
  ta = bitsf(r[0]);
  tb = bitsf(r[1]);
}

// A stage holds one pair of pages, copied HBM -> LDS by the DMA path
// (global_load_lds_dwordx4: lane l writes 16 bytes at stage base + 16 l).
// Every DMA copies from one chunk, so its source is a wave-uniform base plus
// the lane's offset; the chunks' metadata (576 bytes) takes 36 lanes:
//   [   0,1024) K codes page A     [1024,2048) K codes page B
//   [2048,3072) V codes page A     [3072,4096) V codes page B
//   [4096,4608) K scale+zero A     [4608,4672) V scale+zero A
//   [4672,5184) K scale+zero B     [5184,5248) V scale+zero B
//
// With 2-bit pages a stage is:
//   [   0, 512) K codes page A     [ 512,1024) V codes page A
//   [1024,1536) K codes page B     [1536,2048) V codes page B
//   [2048,2560) K scale+zero A     [2560,2624) V scale+zero A
//   [2624,3136) K scale+zero B     [3136,3200) V scale+zero B
// kStages (per code width): the wave reads a stage into registers and
// refills it at once, so the next pairs load while this one is computed.

// Per code width: stage geometry, DMA count, chunk pitch, the query-side
// factor of each K element pair (q_factor), the probability-side factor of
// the second slot group, and the unscale of the odd V tiles; see k_operand /
// k_operand2 / v_operands2. kLazy bounds p (p <= 2^kLazy): the largest V
// scale is (65504 + 65504) / qmax (< 2^13.1 for int4, < 2^15.42 for 2 bits),
// and p * sV must stay below the fp16 maximum 65504 (2^15.999). kLead: a
// column's reference max, when it moves, is set this far above the new
// maximum, so the next move needs a logit kLazy + kLead above that maximum.
template <int kBits>
struct PairFmt;
//
// kQExp: every column's query enters the code products pre-scaled by a power
// of two 2^E with max_d |q_d| 2^E < 2^kQExp. With the 2^-4 slot factor, the
// folded product q 2^E s then stays below 2^(kQExp - 4) times the largest
// fp16 K scale, (65504 + 65504) / qmax rounded to fp16 (8736 for int4,
// 43680 for 2 bits): 34944 and 43680, inside the fp16 range, so no fp16 query
// and K page can overflow it. Small query components keep the resolution of
// fp16's smallest subnormal relative to 2^E instead of to 1.
template <>
struct PairFmt<4> {
  static constexpr int kStageBytes = 5248, kDmaPerStage = 6;
  static constexpr int kQExp = 6;
  static constexpr int kStride = kChunkStride;
  // one stage: deeper rings measured slower (more bytes in flight per wave
  // only queue longer at this rate)
  static constexpr int kStages = 1;
  static constexpr float kPSlot23 = 0.0625f;  // 1/16
  // element pairs 0,1 / 4,5: 2^-4; 2,3 / 6,7: 2^-8
  __device__ static constexpr float q_factor(int j) { return (j & 1) ? 0.00390625f : 0.0625f; }
  static constexpr float kOddTileUnscale = 16777216.0f;  // 2^24, as the even tiles
  static constexpr float kLazy = 2.0f, kLead = 0.0f;
};
template <>
struct PairFmt<2> {
  static constexpr int kStageBytes = 3200, kDmaPerStage = 4;
  static constexpr int kQExp = 4;
  static constexpr int kStride = kK2ChunkStride;
  static constexpr int kStages = 1;
  static constexpr float kPSlot23 = 0.25f;  // 1/4
  // element pair j: 2^-(4 + 2j)
  __device__ static constexpr float q_factor(int j) {
    return j == 0 ? 0.0625f : j == 1 ? 0.015625f : j == 2 ? 0.00390625f : 0.0009765625f;
  }
  static constexpr float kOddTileUnscale = 1048576.0f;  // 2^20
  // p <= 1 (p * sV < 2^15.42); with the lead the reference max moves as
  // rarely as with int4's bound of 4
  static constexpr float kLazy = 0.0f, kLead = 2.0f;
};

// A decode call reads every cache byte once: its loads carry the non-temporal
// policy (nt), which streams them past the caches; on MI355X a pure read of
// 4 KB chunks runs at about 6.8-7.0 TB/s this way against about 6.0 TB/s
// without it. (Column tiles of one sequence read the same pages at about the
// same time, and keep the default policy, so that the caches serve repeats.)
// 16 bytes per lane from base + off (base wave-uniform, held in SGPRs; off the
// lane's 32-bit offset) to LDS at lds_base + 16 * lane, non-temporal. The
// SGPR-base address form costs no 64-bit vector address arithmetic per load
// (the compiler's own lowering of the builtin adds the lane offset to a
// 64-bit VGPR address for every load). The compiler sets M0 (the LDS base)
// for the operand; the s_nop is the wait state between that write and the
// load that reads it.
template <bool kNT = true>
__device__ inline void dma16_at(const uint8_t* base, uint32_t off, uint8_t* lds_base) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint8_t*)(lds_base)));
  if constexpr (kNT) {
    __asm__ __volatile__(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1 nt"
        :
        : "v"(off), "s"(base), "{m0}"(m0)
        : "memory");
  } else {
    __asm__ __volatile__(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(off), "s"(base), "{m0}"(m0)
        : "memory");
  }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// Wait until the oldest stage in flight has landed, when `ahead` later stages
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
// wait for all LDS / scalar-memory operations of this wave
__device__ inline void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }
// the compiler does not know the DMA writes LDS: keep memory accesses on
// their side of the waits
__device__ inline void compiler_fence() { __asm__ __volatile__("" ::: "memory"); }

// The stage a pair occupies, read into registers. The reads are one asm block
// that ends with its own lgkmcnt(0): the compiler cannot see which LDS bytes
// the DMA writes, and for compiler-visible LDS loads it would wait for every
// outstanding DMA, draining the ring; here the caller's explicit vmcnt wait is
// the only guard, and every output is complete when the block ends.
struct PackedStage {
  u4 kcA, kcB, vcA, vcB;     // K / V codes of pages A and B (this lane's 16 bytes)
  u2 sv, zv;                 // V scale / zero of tokens 4g..4g+3 of this column's page
  u4 sc[4];                  // K scale of this lane's 32 channels, this column's page
  u4 ze[4];                  // K zero of this lane's 32 channels, page A for rows c < 8, B above
};

// base: LDS address of the stage; page: this column's page (0 = A, 1 = B);
// zrow: page whose K zeros this lane supplies as row c of the zero-term
// product (0 for c < 8, 1 for c >= 8)
__device__ inline void read_stage_packed(uint32_t base, int lane, int g, int page, int zrow,
                                         PackedStage& r) {
  const uint32_t a_lane = base + 16 * lane;
  const uint32_t a_v = base + 576 * page + 8 * g;
  const uint32_t a_k = base + 576 * page + 16 * g;
  const uint32_t a_z = base + 576 * zrow + 16 * g;
  __asm__ __volatile__(
      "ds_read_b128 %0, %14\n\t"
      "ds_read_b128 %1, %14 offset:1024\n\t"
      "ds_read_b128 %2, %14 offset:2048\n\t"
      "ds_read_b128 %3, %14 offset:3072\n\t"
      "ds_read_b64 %4, %15 offset:4608\n\t"
      "ds_read_b64 %5, %15 offset:4640\n\t"
      "ds_read_b128 %6, %16 offset:4096\n\t"
      "ds_read_b128 %7, %16 offset:4160\n\t"
      "ds_read_b128 %8, %16 offset:4224\n\t"
      "ds_read_b128 %9, %16 offset:4288\n\t"
      "ds_read_b128 %10, %17 offset:4352\n\t"
      "ds_read_b128 %11, %17 offset:4416\n\t"
      "ds_read_b128 %12, %17 offset:4480\n\t"
      "ds_read_b128 %13, %17 offset:4544\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.kcA), "=&v"(r.kcB), "=&v"(r.vcA), "=&v"(r.vcB), "=&v"(r.sv), "=&v"(r.zv),
        "=&v"(r.sc[0]), "=&v"(r.sc[1]), "=&v"(r.sc[2]), "=&v"(r.sc[3]), "=&v"(r.ze[0]),
        "=&v"(r.ze[1]), "=&v"(r.ze[2]), "=&v"(r.ze[3])
      : "v"(a_lane), "v"(a_v), "v"(a_k), "v"(a_z)
      : "memory");
}

// K scale of one page, or (at byte offset 256 past it) K zero
__device__ inline void read_kvec(uint32_t addr, u4 (&v)[4]) {
  __asm__ __volatile__(
      "ds_read_b128 %0, %4 offset:4096\n\t"
      "ds_read_b128 %1, %4 offset:4160\n\t"
      "ds_read_b128 %2, %4 offset:4224\n\t"
      "ds_read_b128 %3, %4 offset:4288\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(addr)
      : "memory");
}

// Both pages' metadata, for groups wider than 8 (every column spans both pages).
struct WideStage {
  u4 kcA, kcB, vcA, vcB;
  u2 svA, zvA, svB, zvB;
  u4 scA[4], scB[4], ze[4];
};
__device__ inline void read_stage_wide(uint32_t base, int lane, int g, int zrow, WideStage& r) {
  const uint32_t a_lane = base + 16 * lane;
  const uint32_t a_v = base + 8 * g;
  __asm__ __volatile__(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:1024\n\t"
      "ds_read_b128 %2, %8 offset:2048\n\t"
      "ds_read_b128 %3, %8 offset:3072\n\t"
      "ds_read_b64 %4, %9 offset:4608\n\t"
      "ds_read_b64 %5, %9 offset:4640\n\t"
      "ds_read_b64 %6, %9 offset:5184\n\t"
      "ds_read_b64 %7, %9 offset:5216\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.kcA), "=&v"(r.kcB), "=&v"(r.vcA), "=&v"(r.vcB), "=&v"(r.svA), "=&v"(r.zvA),
        "=&v"(r.svB), "=&v"(r.zvB)
      : "v"(a_lane), "v"(a_v)
      : "memory");
  read_kvec(base + 16 * g, r.scA);
  read_kvec(base + 576 + 16 * g, r.scB);
  read_kvec(base + 576 * zrow + 256 + 16 * g, r.ze);
}

// The same stages for 2-bit pages: a lane's codes are 8 bytes per page.
struct PackedStage2 {
  u2 kcA, kcB, vcA, vcB;
  u2 sv, zv;
  u4 sc[4];
  u4 ze[4];
};
__device__ inline void read_stage_packed2(uint32_t base, int lane, int g, int page, int zrow,
                                          PackedStage2& r) {
  const uint32_t a_lane = base + 8 * lane;
  const uint32_t a_v = base + 576 * page + 8 * g;
  const uint32_t a_k = base + 576 * page + 16 * g;
  const uint32_t a_z = base + 576 * zrow + 16 * g;
  __asm__ __volatile__(
      "ds_read_b64 %0, %14\n\t"
      "ds_read_b64 %1, %14 offset:1024\n\t"
      "ds_read_b64 %2, %14 offset:512\n\t"
      "ds_read_b64 %3, %14 offset:1536\n\t"
      "ds_read_b64 %4, %15 offset:2560\n\t"
      "ds_read_b64 %5, %15 offset:2592\n\t"
      "ds_read_b128 %6, %16 offset:2048\n\t"
      "ds_read_b128 %7, %16 offset:2112\n\t"
      "ds_read_b128 %8, %16 offset:2176\n\t"
      "ds_read_b128 %9, %16 offset:2240\n\t"
      "ds_read_b128 %10, %17 offset:2304\n\t"
      "ds_read_b128 %11, %17 offset:2368\n\t"
      "ds_read_b128 %12, %17 offset:2432\n\t"
      "ds_read_b128 %13, %17 offset:2496\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.kcA), "=&v"(r.kcB), "=&v"(r.vcA), "=&v"(r.vcB), "=&v"(r.sv), "=&v"(r.zv),
        "=&v"(r.sc[0]), "=&v"(r.sc[1]), "=&v"(r.sc[2]), "=&v"(r.sc[3]), "=&v"(r.ze[0]),
        "=&v"(r.ze[1]), "=&v"(r.ze[2]), "=&v"(r.ze[3])
      : "v"(a_lane), "v"(a_v), "v"(a_k), "v"(a_z)
      : "memory");
}
// K scale of one page, or (at byte offset 256 past it) K zero, 2-bit stage
__device__ inline void read_kvec2(uint32_t addr, u4 (&v)[4]) {
  __asm__ __volatile__(
      "ds_read_b128 %0, %4 offset:2048\n\t"
      "ds_read_b128 %1, %4 offset:2112\n\t"
      "ds_read_b128 %2, %4 offset:2176\n\t"
      "ds_read_b128 %3, %4 offset:2240\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(addr)
      : "memory");
}
struct WideStage2 {
  u2 kcA, kcB, vcA, vcB;
  u2 svA, zvA, svB, zvB;
  u4 scA[4], scB[4], ze[4];
};
__device__ inline void read_stage_wide2(uint32_t base, int lane, int g, int zrow, WideStage2& r) {
  const uint32_t a_lane = base + 8 * lane;
  const uint32_t a_v = base + 8 * g;
  __asm__ __volatile__(
      "ds_read_b64 %0, %8\n\t"
      "ds_read_b64 %1, %8 offset:1024\n\t"
      "ds_read_b64 %2, %8 offset:512\n\t"
      "ds_read_b64 %3, %8 offset:1536\n\t"
      "ds_read_b64 %4, %9 offset:2560\n\t"
      "ds_read_b64 %5, %9 offset:2592\n\t"
      "ds_read_b64 %6, %9 offset:3136\n\t"
      "ds_read_b64 %7, %9 offset:3168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.kcA), "=&v"(r.kcB), "=&v"(r.vcA), "=&v"(r.vcB), "=&v"(r.svA), "=&v"(r.zvA),
        "=&v"(r.svB), "=&v"(r.zvB)
      : "v"(a_lane), "v"(a_v)
      : "memory");
  read_kvec2(base + 16 * g, r.scA);
  read_kvec2(base + 576 + 16 * g, r.scB);
  read_kvec2(base + 576 * zrow + 256 + 16 * g, r.ze);
}
__device__ inline void read_packed(uint32_t base, int lane, int g, int page, int zrow, PackedStage& r) {
  read_stage_packed(base, lane, g, page, zrow, r);
}
__device__ inline void read_packed(uint32_t base, int lane, int g, int page, int zrow, PackedStage2& r) {
  read_stage_packed2(base, lane, g, page, zrow, r);
}
__device__ inline void read_wide(uint32_t base, int lane, int g, int zrow, WideStage& r) {
  read_stage_wide(base, lane, g, zrow, r);
}
__device__ inline void read_wide(uint32_t base, int lane, int g, int zrow, WideStage2& r) {
  read_stage_wide2(base, lane, g, zrow, r);
}

// units of a sequence: its full pages, plus one for a non-empty tail
__device__ inline int units_of(int ctx, int max_pages) {
  ctx = min(ctx, max_pages * kPage);
  if (ctx <= 0) return 0;
  return ctx / kPage + ((ctx % kPage) ? 1 : 0);
}

// Multi-query column tiles: when a sequence's new tokens need more than 16
// matrix-core columns per KV head, they are cut into tiles of tpt whole
// tokens, and tile k of sequence b is streamed as its own virtual sequence
// bv = b * ct_n + k. Its columns are tokens [k tpt, k tpt + tpt) of b's
// new tokens, which see the cache positions up to the tile's last token, so
// the tile needs only the pages (and the tail, if it reaches it) holding
// those positions; a tile past the sequence's token count has no units.
// Returns the full pages and tail tokens the virtual sequence streams.
struct VSpan {
  int full, tail;
};
__device__ inline VSpan tile_span(int bv, const int32_t* ctx_lens, int max_pages,
                                  const int32_t* cu_q, int ct_n, int tpt) {
  const int b = bv / ct_n;
  const int ctx = min(ctx_lens[b], max_pages * kPage);
  if (ctx <= 0) return {0, 0};
  const int tb = cu_q[b + 1] - cu_q[b];
  const int t0 = (bv - b * ct_n) * tpt;
  if (t0 >= tb) return {0, 0};
  const int len = min(ctx, max(1, ctx - tb + min(tb, t0 + tpt)));  // positions 0 .. len - 1
  const int full = ctx / kPage;
  if (len <= full * kPage) return {(len + kPage - 1) / kPage, 0};
  return {full, ctx % kPage};
}

// The wave that owns unit u when U units are split into W ranges
// [w*U/W, (w+1)*U/W): the largest w with floor(w*U/W) <= u.
__device__ __host__ inline int owner_wave(int64_t u, int64_t U, int W) {
  return static_cast<int>(((u + 1) * W - 1) / U);
}

// Partial results: one slot of G x (128 outputs, m, l) floats per
// (b*Hkv + h, wave) pair, at slot index (b*Hkv + h) + wave.
constexpr int kSlotStride = kHeadDim + 4;  // 128 outputs, m, l, 2 pad (16-byte rows)

// G is the number of matrix-core columns one KV head feeds. For decode it is
// the query group Hq / Hkv. With kMQ (several query tokens per sequence) a
// column is a (query token, query head) pair: G = max_q * gq columns, column v
// holds token v / gq and head v % gq of the group, and attends causally: token
// t of the T_b new tokens of sequence b sits at position ctx_b - T_b + t and
// sees the cache positions up to it.
//
// kAppend (int4 decode only): the call first appends one token per sequence,
// the token at cache position ctx_b - 1, from k_new / v_new [B][Hkv][128]. The
// wave that owns the last unit of a (b, h) does that append: it stores the
// token in the fp16 tail, or, when the token completes a page, quantizes the
// page (15 tail tokens and the new one) into the pool and into its ring stage.
// Either way it attends over the new token straight from its inputs.
// Waves per SIMD: two, or three with 2-bit codes, whose pairs carry fewer
// bytes for the same instruction count (the 2-bit kernel fits 168 VGPRs),
// and with more than 8 multi-query columns, whose longer pair path hides
// better behind a third wave (168 VGPRs; its few spills sit outside the pair
// loop). The launches size the grid to match (stream_waves).
constexpr int waves_per_simd(int G, bool kMQ, int kBits) {
  return (kBits == 2 || (kMQ && G > 8)) ? 3 : 2;
}
template <int G, bool kMQ, int kBits, bool kAppend>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(waves_per_simd(G, kMQ, kBits),
                                                                     waves_per_simd(G, kMQ, kBits)))) void decode_stream_kernel(
    const __half* __restrict__ q, uint8_t* __restrict__ pages,
    __half* __restrict__ tail_k, __half* __restrict__ tail_v,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens,
    int32_t* __restrict__ total_units, int2* __restrict__ seg_waves, int32_t B, int32_t max_pages,
    int32_t hkv, float sm_scale, float* __restrict__ slots, const int32_t* __restrict__ cu_q,
    int32_t gq, int32_t total_q, const __half* __restrict__ k_new, const __half* __restrict__ v_new,
    int32_t ct_n, int32_t tpt) {
  static_assert(!kAppend || (kBits == 4 && !kMQ), "the fused append serves the int4 decode");
  constexpr bool kPacked = (G <= 8);    // columns split between the two pages of a pair
  constexpr bool kHiLoCols = (G <= 4);  // and between the hi / lo parts of the output operand
  const int w = blockIdx.x, W = gridDim.x;
  const int lane = threadIdx.x;
  const int c = lane & 15, g = lane >> 4;
  const int hq = hkv * (kMQ ? gq : G);
  using PF = PairFmt<kBits>;
  constexpr int kStages = PF::kStages;
  using PStage = std::conditional_t<kBits == 4, PackedStage, PackedStage2>;
  using WStage = std::conditional_t<kBits == 4, WideStage, WideStage2>;
  // kMQ: B counts virtual sequences (column tiles, see tile_span); the real
  // sequence of virtual sequence b is b / ct_n
  auto span_of = [&](int b) -> VSpan {
    if constexpr (kMQ) {
      return tile_span(b, ctx_lens, max_pages, cu_q, ct_n, tpt);
    } else {
      const int ctx = min(ctx_lens[b], max_pages * kPage);
      return ctx > 0 ? VSpan{ctx / kPage, ctx % kPage} : VSpan{0, 0};
    }
  };
  auto nunits_of = [&](int b) {
    const VSpan v = span_of(b);
    return v.full + (v.tail ? 1 : 0);
  };
  auto real_seq = [&](int b) { return kMQ ? b / ct_n : b; };

  // ---- unit plan ----
  // units(b) = full pages of b plus one for a non-empty tail; (b, h) pairs are
  // laid out b-major, so sequence b's units start at Hkv * sum_{b' < b} units(b').
  // Every wave derives the total and its own start from ctx_lens. The wave
  // that owns the first unit of a (b, h) records which waves share it.
  int64_t U;
  {
    int local = 0;
    for (int b = lane; b < B; b += 64) local += nunits_of(b);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
    // every lane holds the sum; readfirstlane tells the compiler it is
    // wave-uniform, so the range and cursor arithmetic stays scalar
    U = (int64_t)hkv * __builtin_amdgcn_readfirstlane(local);
  }
  // Unit indices fit in int32 (the host checks B * Hkv * (max_pages + 1)), so
  // the cursors count in 32 bits and every per-pair range check is one scalar
  // compare. The 64-bit divisions run on the vector unit; readfirstlane brings
  // the results back to scalar registers.
  const int32_t u0 = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((int64_t)w * U / W));
  const int32_t u1 = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((int64_t)(w + 1) * U / W));
  const bool has_range = u0 < u1;
  if (w == 0 && lane == 0) total_units[0] = static_cast<int32_t>(U);
  if (!has_range) return;
  const int nchunks = (B + 63) / 64;
  int b0 = -1;
  int32_t s0 = 0;  // first unit of sequence b0
  {
    int64_t carry = 0;
    for (int k = 0; k < nchunks && b0 < 0; ++k) {
      const int b = 64 * k + lane;
      const int n = (b < B) ? nunits_of(b) : 0;
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

  // Column roles (c = lane % 16):
  //   G <= 4: c = 8*part + 4*page + hh  (part 0 / 1 = high / low fp16 part of
  //           the output operand; page 0 / 1 = page A / B of a pair)
  //   G <= 8: c = 8*page + hh
  //   G > 8:  c = hh, both pages in every column
  // with query head hh of the group; hh >= G are padding columns that repeat
  // head hh % G so every value they carry stays finite.
  const int hh = kHiLoCols ? (c & 3) : (kPacked ? (c & 7) : c);
  const int head = hh % G;
  const int pslot = kHiLoCols ? ((c >> 2) & 1) : (kPacked ? (c >> 3) : 0);
  const bool lo_col = kHiLoCols && c >= 8;
  const int zrow = c >> 3;  // page of the K zeros this lane supplies (zero-term product)
  const float l2s = sm_scale * kLog2e;  // logits go to log2 units
  const float qk_scale = l2s * kQkUnscale;
  float qk_col = qk_scale;  // qk_scale / 2^E for the column's query pre-scale 2^E

  // ---- cursors over the wave's units (all fields wave-uniform) ----
  struct Cursor {
    int32_t u;   // flat index of the next unit
    int b, h;    // sequence, KV head
    int unit;    // unit inside (b, h)
    int full;    // full pages of b
    int nunits;  // units of b
    int tail;    // tokens in the fp16 tail of b
  };
  auto seq_info = [&](int b, Cursor& cu) {
    const VSpan v = span_of(b);
    cu.full = v.full;
    cu.tail = v.tail;
    cu.nunits = cu.full + (cu.tail ? 1 : 0);
  };
  Cursor start;
  {
    start.u = u0;
    start.b = b0;
    seq_info(b0, start);
    const int32_t local = u0 - s0;
    start.h = local / start.nunits;
    start.unit = local % start.nunits;
  }
  auto advance = [&](Cursor& cu, int n_units) {
    cu.u += n_units;
    cu.unit += n_units;
    if (cu.unit >= cu.nunits && cu.u < u1) {
      cu.unit = 0;
      if (++cu.h == hkv) {
        cu.h = 0;
        do { ++cu.b; seq_info(cu.b, cu); } while (cu.nunits == 0);
      }
    }
  };

  // ---- DMA ring ----
  __shared__ __align__(16) uint8_t stage_s[kStages][PF::kStageBytes];
  __shared__ __align__(16) _Float16 tail_s[kPage][kHeadDim];  // fp16 tail V, one (b, h) at a time
  // kAppend: the raw K rows (bytes 0..4095) and V rows (4096..8191) of a page
  // the new token completes: 15 tail rows and the new token as row 15
  __shared__ __align__(16) uint8_t raw_s[kAppend ? 2 * kPage * 2 * kHeadDim : 16];
  Cursor prod = start;
  int issued = 0, consumed = 0;
  int pstage = 0, cstage = 0;  // ring slots of the next issue / the next consume
  // kMQ: the column's causal limit (cache position) in the current segment
  int col_lim = 0;
  // kMQ: the smallest limit among the wave's columns (its tile's first
  // token), wave-uniform: a pair whose positions all lie at or below it
  // needs no mask
  int lim_min = 0;
  auto q_row = [&](int bv, int h) {
    if constexpr (kMQ) {
      // a sequence with fewer new tokens than columns repeats its last token
      // in the spare columns (their results are not stored)
      const int b = real_seq(bv);
      const int ctx = min(ctx_lens[b], max_pages * kPage);
      const int q0 = cu_q[b], tb = cu_q[b + 1] - q0;
      const int t = min((bv - b * ct_n) * tpt + head / gq, max(tb - 1, 0));
      col_lim = ctx - tb + t;
      lim_min = ctx - tb + min((bv - b * ct_n) * tpt, max(tb - 1, 0));
      const int64_t row = min(max((int64_t)q0 + t, (int64_t)0), (int64_t)total_q - 1);
      return reinterpret_cast<const uint8_t*>(q + (row * hq + h * gq + head % gq) * kHeadDim);
    } else {
      return reinterpret_cast<const uint8_t*>(q + ((int64_t)bv * hq + h * G + head) * kHeadDim);
    }
  };
  // Block ids of the pair at the producer cursor, loaded one pair ahead of
  // their use so the scalar-load latency overlaps a whole iteration. A single
  // page is fetched twice (as pages A and B) so the stage never holds stale
  // scales.
  // Producer state kept per segment, so that a pair inside a segment costs a
  // compare, two id loads and the chunk addresses: the end of the segment's
  // full pages within the range, the segment's block-table row and the base
  // of its KV head's chunks.
  bool p_live = false;
  int p_page_end = 0;
  const int32_t* p_row = block_table;
  const uint8_t* p_base = pages;
  // chunk (id, h) is at pages + (id * Hkv + h) * stride; id * Hkv + h <
  // num_pages * Hkv fits in 32 bits
  const uint32_t id_stride = static_cast<uint32_t>(hkv) * PF::kStride;
  int nid_a = 0, nid_b = 0;
  auto p_ids = [&]() {
    // Both ids load unconditionally (the second index clamped to the row) and
    // the pair / single choice is made where they are used, one pair later,
    // so nothing waits for these scalar loads here.
    nid_a = p_row[prod.unit];
    nid_b = p_row[min(prod.unit + 1, max_pages - 1)];
  };
  // from the cursor (a unit of the range, possibly a tail or the end of a
  // segment), on to the next full page in the range
  auto p_seek = [&]() {
    if (prod.u < u1 && prod.unit >= prod.nunits) advance(prod, 0);
    while (prod.u < u1 && prod.unit >= prod.full) advance(prod, 1);
    p_live = prod.u < u1;
    if (!p_live) return;
    p_page_end = min(prod.full, prod.unit + (u1 - prod.u));
    // B * max_pages fits in int32 (the host checks B * Hkv * (max_pages + 1))
    p_row = block_table + real_seq(prod.b) * max_pages;
    p_base = pages + static_cast<uint64_t>(static_cast<uint32_t>(prod.h)) * PF::kStride;
    p_ids();
  };
  // Issue the pair at the producer cursor (tails need no DMA).
  auto produce = [&]() {
    if (!p_live) return;
    const int np = (prod.unit + 1 < p_page_end) ? 2 : 1;
    // the ids are wave-uniform (scalar loads at a uniform address); saying
    // so keeps the chunk bases in scalar registers, as the DMA form needs
    const int idA = __builtin_amdgcn_readfirstlane(nid_a);
    const int idB = __builtin_amdgcn_readfirstlane((np == 2) ? nid_b : nid_a);
    const uint8_t* chA = p_base + static_cast<uint64_t>(static_cast<uint32_t>(idA)) * id_stride;
    const uint8_t* chB = p_base + static_cast<uint64_t>(static_cast<uint32_t>(idB)) * id_stride;
    uint8_t* st = stage_s[pstage];
    if (++pstage == kStages) pstage = 0;
    const uint32_t lo = 16u * static_cast<uint32_t>(lane);
    if constexpr (kBits == 4) {
      auto issue = [&](auto nt) {
        constexpr bool kNT = decltype(nt)::value;
        dma16_at<kNT>(chA, lo + kOffKCodes, st + 0);
        dma16_at<kNT>(chB, lo + kOffKCodes, st + 1024);
        dma16_at<kNT>(chA, lo + kOffVCodes, st + 2048);
        dma16_at<kNT>(chB, lo + kOffVCodes, st + 3072);
        if (lane < 36) {
          dma16_at<kNT>(chA, lo + kOffKScale, st + 4096);
          dma16_at<kNT>(chB, lo + kOffKScale, st + 4672);
        }
      };
      // several column tiles per sequence: the default policy (see dma16_at)
      if (kMQ && ct_n > 1)
        issue(std::false_type{});
      else
        issue(std::true_type{});
    } else {
      dma16_at(chA, lo, st + 0);
      dma16_at(chB, lo, st + 1024);
      if (lane < 36) {
        dma16_at(chA, lo + kOff2KScale, st + 2048);
        dma16_at(chB, lo + kOff2KScale, st + 2624);
      }
    }
    if constexpr (kAppend) {
      // the entry ends with the page the new token completes: bring its 15
      // tail rows and the new token along with the stage, so the page is
      // quantized from LDS when the entry is consumed (issued with the stage
      // and before any later one, these loads are covered by its wait)
      if (prod.tail == 0 && prod.unit + np == prod.full) {
        const int64_t bh = (int64_t)prod.b * hkv + prod.h;
        const uint8_t* tk = reinterpret_cast<const uint8_t*>(tail_k + bh * kPage * kHeadDim);
        const uint8_t* tv = reinterpret_cast<const uint8_t*>(tail_v + bh * kPage * kHeadDim);
        const uint8_t* kn = reinterpret_cast<const uint8_t*>(k_new + bh * kHeadDim);
        const uint8_t* vn = reinterpret_cast<const uint8_t*>(v_new + bh * kHeadDim);
        constexpr int kRow = 2 * kHeadDim;  // bytes per token row
#pragma unroll
        for (int i = 0; i < 3; ++i) {
          dma16_at(tk, lo + 1024 * i, raw_s + 1024 * i);
          dma16_at(tv, lo + 1024 * i, raw_s + kPage * kRow + 1024 * i);
        }
        if (lane < 48) {  // rows 12..14
          dma16_at(tk, lo + 3072, raw_s + 3072);
          dma16_at(tv, lo + 3072, raw_s + kPage * kRow + 3072);
        }
        if (lane < 16) {  // the new token, row 15
          dma16_at(kn, lo, raw_s + (kPage - 1) * kRow);
          dma16_at(vn, lo, raw_s + kPage * kRow + (kPage - 1) * kRow);
        }
      }
    }
    ++issued;
    prod.u += np;
    prod.unit += np;
    if (prod.unit < p_page_end) p_ids();
    else p_seek();
  };

  // ---- per-(b, h) state, per column ----
  h8 qc[4];  // query of the column's head, pre-scaled for the code operands
  h8 qh[4];  // the same query, plain (zero-point term)
  float m_run = kMEmpty, l_part = 0.f, lz_part = 0.f;
  f4 o[8];
  int cur_b = -1, cur_h = 0;
  // unscale of the page products accumulated in output tile t
  auto tile_unscale = [](int t) { return (t & 1) ? PF::kOddTileUnscale : kPvUnscale; };

  auto begin_segment = [&](const Cursor& cu) {
    const int b = cu.b, h = cu.h;
    cur_b = b;
    cur_h = h;
    // the owner of the segment's first unit records the waves sharing it
    const int32_t first = cu.u - cu.unit;
    if (first >= u0 && lane == 0)
      seg_waves[(int64_t)b * hkv + h] = make_int2(owner_wave(first, U, W), owner_wave(first + cu.nunits - 1, U, W));
    // the query of the new (b, h); loading it waits for the ring's DMAs,
    // once per segment
    u4 raw[4];
    const uint8_t* qr = q_row(b, h);
#pragma unroll
    for (int m = 0; m < 4; ++m) raw[m] = ld16(qr + 2 * (32 * m + 8 * g));
    // the column's pre-scale 2^E: E = kQExp - e with max_d |q_d| = f 2^e,
    // f in [0.5, 1), so max |q| 2^E < 2^kQExp (E in [-10, 29] for fp16 q;
    // a zero query gives E = kQExp)
    float amax = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const h8 v = as_h8(raw[m]);
      qh[m] = v;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(static_cast<float>(v[i])));
    }
    const int E = PF::kQExp - __builtin_amdgcn_frexp_expf(rows_max(amax));
    const float pre = __builtin_bit_cast(float, static_cast<uint32_t>(127 + E) << 23);
    qk_col = qk_scale * __builtin_bit_cast(float, static_cast<uint32_t>(127 - E) << 23);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // element i of product m is channel 32m+8g+i, pre-scaled by 2^E times
      // the factor of its element pair i / 2
#pragma unroll
      for (int i = 0; i < 8; ++i)
        qc[m][i] = static_cast<_Float16>(static_cast<float>(qh[m][i]) * pre * PF::q_factor(i >> 1));
    }
    m_run = kMEmpty;
    l_part = 0.f;
    lz_part = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = f4{0.f, 0.f, 0.f, 0.f};
  };

  // Partial-result stores wait for nothing, but while they are outstanding
  // they hold vmcnt, so the ring's next waits would stall on them (their
  // write-back is slow under a full read stream). A packed layout therefore
  // keeps a finished segment's partial in registers and writes it when the
  // next segment ends, or when the range is done -- for most waves, after the
  // last ring wait. After the page merge every head's values sit in
  // kCopies columns, so each copy keeps a different 1/kCopies of the outputs.
  constexpr int kCopies = kHiLoCols ? 4 : 2;  // columns holding the same head
  constexpr int kKeep = 8 / kCopies;          // output tiles kept per lane
  // kept tile n is output tile kKeep * copy + n, of the parity of n
  static_assert(kKeep % 2 == 0, "kept tiles keep their parity");
  const int copy = kHiLoCols ? (c >> 2) : (c >> 3);
  const int head_col = kHiLoCols ? (c & 3) : (c & 7);
  f4 keep_o[kKeep];
  float keep_m = 0.f, keep_l = 0.f;
  int64_t keep_slot = -1;  // wave-uniform; -1 when nothing is held
  auto store_kept = [&]() {
    if (keep_slot < 0) return;
    if (head_col < G) {
      float* dst = slots + (keep_slot * G + head_col) * kSlotStride;
#pragma unroll
      for (int n = 0; n < kKeep; ++n)
        *reinterpret_cast<f4*>(dst + 16 * (kKeep * copy + n) + 4 * g) = keep_o[n];
      if (g == 0 && copy == 0) { dst[kHeadDim] = keep_m; dst[kHeadDim + 1] = keep_l; }
    }
    keep_slot = -1;
  };

  auto end_segment = [&]() {
    float l = rows_sum(l_part), lz = rows_sum(lz_part);
    float m_out = m_run;
    f4 ov[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) ov[t] = o[t];
    const int64_t slot = (int64_t)cur_b * hkv + cur_h + w;
    if constexpr (kPacked) {
      if constexpr (kHiLoCols) {
        // high + low parts: same logits, same maximum, columns c and c ^ 8
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) ov[t][i] += xor8(ov[t][i]);
      }
      // pages A and B of the pairs kept their own maxima: merge the two columns
      auto partner = [&](float v) { return kHiLoCols ? xor4(v, c) : xor8(v); };
      const float M = fmaxf(m_run, partner(m_run));
      const float a = __builtin_amdgcn_exp2f(m_run - M);
      l *= a;
      lz *= a;
      l += partner(l);
      lz += partner(lz);
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = ov[t][i] * a;
          ov[t][i] = v + partner(v);
        }
      m_out = M;
      // write the partial held from an earlier segment, hold this one
      store_kept();
#pragma unroll
      for (int n = 0; n < kKeep; ++n) {
        f4 v = ov[n];
#pragma unroll
        for (int k = 1; k < kCopies; ++k)
          if (copy == k) v = ov[kKeep * k + n];
#pragma unroll
        for (int i = 0; i < 4; ++i) keep_o[n][i] = v[i] * tile_unscale(n) + lz;
      }
      keep_m = m_out;
      keep_l = l;
      keep_slot = slot;
    } else {
      if (c < G) {
        float* dst = slots + (slot * G + c) * kSlotStride;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          f4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = ov[t][i] * tile_unscale(t) + lz;
          *reinterpret_cast<f4*>(dst + 16 * t + 4 * g) = v;
        }
        if (g == 0) { dst[kHeadDim] = m_out; dst[kHeadDim + 1] = l; }
      }
    }
  };

  // The reference max of a column moves only when a logit passes it by more
  // than PF::kLazy (log2 units), so most pages skip rescaling the
  // accumulators; a probability is then at most 2^PF::kLazy, which keeps
  // p * sV inside the fp16 range for every fp16 V scale.
  auto rescale_to = [&](float mb) {
    const bool up = mb > m_run + PF::kLazy;
    if (__any(up)) {
      const float mnew = up ? (PF::kLead != 0.f ? mb + PF::kLead : mb) : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);
      l_part *= alpha;
      lz_part *= alpha;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[t] *= alpha;
      m_run = mnew;
    }
  };

  // ---- fp16 tail of (cur_b, cur_h): logits and output products on fp16 values;
  // in packed layouts only page-A columns take it
  // tail_pos0: cache position of the tail's first token
  auto process_tail = [&](int tail_n, int tail_pos0) {
    const int64_t bh = (int64_t)real_seq(cur_b) * hkv + cur_h;
    const uint8_t* tk = reinterpret_cast<const uint8_t*>(tail_k + bh * kPage * kHeadDim);
    const uint8_t* tv = reinterpret_cast<const uint8_t*>(tail_v + bh * kPage * kHeadDim);
    // kAppend: the new token is tail slot tail_n - 1; it is read from the
    // inputs (its tail store below is not ordered before this wave's loads)
    const int slot_new = kAppend ? tail_n - 1 : -1;
    const uint8_t* kn = nullptr;
    const uint8_t* vn = nullptr;
    if constexpr (kAppend) {
      kn = reinterpret_cast<const uint8_t*>(k_new + bh * kHeadDim);
      vn = reinterpret_cast<const uint8_t*>(v_new + bh * kHeadDim);
      // lanes 0..15 store its K row, lanes 16..31 its V row, 16 bytes each
      if (lane < 32) {
        __half* row = (lane < 16 ? tail_k : tail_v) + (bh * kPage + slot_new) * kHeadDim;
        *reinterpret_cast<u4*>(reinterpret_cast<uint8_t*>(row) + 16 * (lane & 15)) =
            ld16((lane < 16 ? kn : vn) + 16 * (lane & 15));
      }
    }
    _Float16 (*tv_s)[kHeadDim] = tail_s;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int piece = lane + 64 * i;  // 16-byte piece of the 16 x 256-byte rows
      const uint8_t* src = (kAppend && (piece >> 4) == slot_new) ? vn + 16 * (piece & 15) : tv + 16 * piece;
      reinterpret_cast<u4*>(&tv_s[0][0])[piece] = ld16(src);
    }
    // logits: A = K tail values (token c, channels 32m+8g..+8), B = plain q
    const uint8_t* krow = (kAppend && c == slot_new) ? kn : tk + 2 * c * kHeadDim;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) acc = mfma(as_h8(ld16(krow + 2 * (32 * m + 8 * g))), qh[m], acc);
    float lg[4];
    float mb = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bool ok = 4 * g + i < tail_n && pslot == 0;
      if constexpr (kMQ) ok = ok && tail_pos0 + 4 * g + i <= col_lim;
      lg[i] = ok ? acc[i] * l2s : kNegInf;
      mb = fmaxf(mb, lg[i]);
    }
    mb = rows_max(mb);
    rescale_to(mb);
    const float ms = m_run;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(lg[i] - ms);
      l_part += p[i];
    }
    __builtin_amdgcn_wave_barrier();
    // output: A = V tail values of tokens 4g..4g+3 (slots 0..3), slots 4..7 empty
    h8 bhi, blo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = (i < 4) ? p[i] : 0.f;
      const _Float16 xh = static_cast<_Float16>(x);
      bhi[i] = xh;
      blo[i] = static_cast<_Float16>(x - static_cast<float>(xh));
    }
    const h8 bsel = lo_col ? blo : bhi;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      h8 a;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = (4 * g + i < tail_n) ? tv_s[4 * g + i][16 * t + c] : static_cast<_Float16>(0.f);
        a[4 + i] = static_cast<_Float16>(0.f);
      }
      f4 ot = {0.f, 0.f, 0.f, 0.f};
      if constexpr (kHiLoCols) {
        ot = mfma(a, bsel, ot);
      } else {
        ot = mfma(a, bhi, ot);
        ot = mfma(a, blo, ot);
      }
      // bring the tail's products to the pages' scale for tile t (exact)
      o[t] += ot * (1.0f / tile_unscale(t));
    }
    __builtin_amdgcn_wave_barrier();
  };

  // ---- one pair of pages from a ring stage ----
  auto lds_addr = [&](const uint8_t* p) -> uint32_t {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) uint8_t*)(p)));
  };
  // The stage just read into registers (its asm block ended with
  // lgkmcnt(0)) is free: refill it with the next pair at once, so kStages
  // pairs are in flight while this one is computed.
  auto refill = [&]() {
    compiler_fence();
    produce();
    compiler_fence();
  };
  // fp16 (hi, lo) parts of x = p * s for output slot k (slots 2,3,6,7 carry
  // 1/16, applied to p: an exact power-of-2 scaling, so the product is the
  // same, and s enters the mixed-precision fma as fp16 unconverted)
  auto ps_split = [&](float pk, _Float16 s, int k, _Float16& hi, _Float16& lo) {
    const float pf = pk * (((k & 2) == 0) ? 1.0f : PF::kPSlot23);
    const float sv = static_cast<float>(s);
    hi = static_cast<_Float16>(__builtin_fmaf(pf, sv, 0.0f));
    lo = static_cast<_Float16>(__builtin_fmaf(pf, sv, -static_cast<float>(hi)));
  };
  // pos0: cache position of page A's first token
  auto process_pair = [&](const uint8_t* st, bool has_b, int pos0) {
    f4 accA = {0.f, 0.f, 0.f, 0.f}, accB = {0.f, 0.f, 0.f, 0.f};
    if constexpr (kPacked) {
      PStage r;
      read_packed(lds_addr(st), lane, g, pslot, zrow, r);
      refill();
      // ---- logits of this column's page (K scale of that page in the operand) ----
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        h8 hi, lo;
        qs_split(qc[m], r.sc[m], hi, lo);
        const h8 ka = k_op(r.kcA, m);
        const h8 kb = k_op(r.kcB, m);
        accA = mfma(ka, hi, accA);
        accA = mfma(ka, lo, accA);
        accB = mfma(kb, hi, accB);
        accB = mfma(kb, lo, accB);
      }
      float za, zb;
      zero_terms(qh, r.ze, za, zb);
      const float zl = (pslot && !has_b) ? kNegInf : (pslot ? zb : za) * l2s;
      const f4 mine = pslot ? accB : accA;
      float lg[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) lg[k] = mine[k] * qk_col + zl;
      if constexpr (kMQ) {
        if (pos0 + 2 * kPage - 1 > lim_min) {
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (pos0 + kPage * pslot + 4 * g + k > col_lim) lg[k] = kNegInf;
        }
      }
      const float mb = rows_max(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])));
      rescale_to(mb);
      const float ms = m_run;
      _Float16 hv[4], lv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float pk = __builtin_amdgcn_exp2f(lg[k] - ms);
        l_part += pk;
        lz_part += pk * static_cast<float>(h_at2(r.zv, k));
        ps_split(pk, h_at2(r.sv, k), k, hv[k], lv[k]);
      }
      // this column's page occupies slots 0..3 (page A) or 4..7 (page B)
      auto place = [&](const _Float16 (&x)[4]) -> h8 {
        const uint32_t d0 = __builtin_bit_cast(uint32_t, h2v{x[0], x[1]});
        const uint32_t d1 = __builtin_bit_cast(uint32_t, h2v{x[2], x[3]});
        u4 v;
        v[0] = pslot ? 0u : d0;
        v[1] = pslot ? 0u : d1;
        v[2] = pslot ? d0 : 0u;
        v[3] = pslot ? d1 : 0u;
        return as_h8(v);
      };
      if constexpr (kHiLoCols) {
        _Float16 sel[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) sel[k] = lo_col ? lv[k] : hv[k];
        const h8 b = place(sel);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          h8 ve, vo;
          v_ops(r.vcA, r.vcB, m, ve, vo);
          o[2 * m] = mfma(ve, b, o[2 * m]);
          o[2 * m + 1] = mfma(vo, b, o[2 * m + 1]);
        }
      } else {
        const h8 bh = place(hv), bl = place(lv);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          h8 ve, vo;
          v_ops(r.vcA, r.vcB, m, ve, vo);
          o[2 * m] = mfma(ve, bh, o[2 * m]);
          o[2 * m] = mfma(ve, bl, o[2 * m]);
          o[2 * m + 1] = mfma(vo, bh, o[2 * m + 1]);
          o[2 * m + 1] = mfma(vo, bl, o[2 * m + 1]);
        }
      }
    } else {
      WStage r;
      read_wide(lds_addr(st), lane, g, zrow, r);
      refill();
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        h8 hi, lo;
        qs_split(qc[m], r.scA[m], hi, lo);
        const h8 ka = k_op(r.kcA, m);
        accA = mfma(ka, hi, accA);
        accA = mfma(ka, lo, accA);
        qs_split(qc[m], r.scB[m], hi, lo);
        const h8 kb = k_op(r.kcB, m);
        accB = mfma(kb, hi, accB);
        accB = mfma(kb, lo, accB);
      }
      float zA, zB;
      zero_terms(qh, r.ze, zA, zB);
      const float zlB = has_b ? zB * l2s : kNegInf;
      float lgA[4], lgB[4];
      float mb = kNegInf;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lgA[k] = accA[k] * qk_col + zA * l2s;
        lgB[k] = accB[k] * qk_col + zlB;
      }
      if constexpr (kMQ) {
        if (pos0 + 2 * kPage - 1 > lim_min) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (pos0 + 4 * g + k > col_lim) lgA[k] = kNegInf;
            if (pos0 + kPage + 4 * g + k > col_lim) lgB[k] = kNegInf;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) mb = fmaxf(mb, fmaxf(lgA[k], lgB[k]));
      mb = rows_max(mb);
      rescale_to(mb);
      const float msw = m_run;
      h8 bhi, blo;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float pa = __builtin_amdgcn_exp2f(lgA[k] - msw);
        const float pb = __builtin_amdgcn_exp2f(lgB[k] - msw);
        l_part += pa + pb;
        lz_part += pa * static_cast<float>(h_at2(r.zvA, k)) + pb * static_cast<float>(h_at2(r.zvB, k));
        _Float16 h, l;
        ps_split(pa, h_at2(r.svA, k), k, h, l);
        bhi[k] = h;
        blo[k] = l;
        ps_split(pb, h_at2(r.svB, k), k + 4, h, l);
        bhi[k + 4] = h;
        blo[k + 4] = l;
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        h8 ve, vo;
        v_ops(r.vcA, r.vcB, m, ve, vo);
        o[2 * m] = mfma(ve, bhi, o[2 * m]);
        o[2 * m] = mfma(ve, blo, o[2 * m]);
        o[2 * m + 1] = mfma(vo, bhi, o[2 * m + 1]);
        o[2 * m + 1] = mfma(vo, blo, o[2 * m + 1]);
      }
    }
  };

  // ---- main stream ----
  // kStages pairs are issued ahead. vmcnt counts this wave's outstanding
  // vector-memory operations and loads complete in issue order, so "at most
  // 6 x (pairs issued after this one)" outstanding means this pair has landed
  // in LDS; other outstanding operations (query and tail loads,
  // partial-result stores) can only make the wait stricter.
  // kAppend, a (b, h) whose new token completes page P: quantize P from its
  // raw rows (in LDS with the stage), store it in the pool, and put it into
  // the stage in place of the copy the DMA brought from the pool (page B of
  // a pair, or both copies of a single page). The tail's LDS area is the
  // scratch for the codes.
  auto fresh_page = [&](uint8_t* st, bool pair, int P) {
    const __half* rk = reinterpret_cast<const __half*>(raw_s);
    const __half* rv = reinterpret_cast<const __half*>(raw_s + kPage * 2 * kHeadDim);
    auto krow = [&](int t) { return rk + t * kHeadDim; };
    auto vrow = [&](int t) { return rv + t * kHeadDim; };
    uint8_t (*scr)[kHeadDim] = reinterpret_cast<uint8_t (*)[kHeadDim]>(&tail_s[0][0]);
    PageShare<4> sh;
    auto none = [](const PageShare<4>&) {};
    quantize_page<4>(krow, vrow, lane, scr, scr + kPage, sh, none, none);
    const int32_t id = block_table[cur_b * max_pages + P];
    store_page<4>(pages + static_cast<uint64_t>(static_cast<uint32_t>(id * hkv + cur_h)) * PF::kStride,
                  lane, sh, true);
    auto to_stage = [&](int which) {
      *reinterpret_cast<uint4*>(st + 1024 * which + 16 * lane) = sh.kcode;
      *reinterpret_cast<uint4*>(st + 2048 + 1024 * which + 16 * lane) = sh.vcode;
      uint8_t* meta = st + 4096 + 576 * which;
      reinterpret_cast<__half2*>(meta)[lane] = sh.ks;
      reinterpret_cast<__half2*>(meta + (kOffKZero - kOffKScale))[lane] = sh.kz;
      if ((lane & 3) == 0) {
        reinterpret_cast<__half*>(meta + (kOffVScale - kOffKScale))[lane >> 2] = sh.vs;
        reinterpret_cast<__half*>(meta + (kOffVZero - kOffKScale))[lane >> 2] = sh.vz;
      }
    };
    to_stage(1);
    if (!pair) to_stage(0);
    wait_lgkmcnt0();
  };
  auto consume_pair = [&](int np, int pos0, int fresh_p) {
    wait_pages_after<PF::kDmaPerStage, kStages - 1>(issued - consumed - 1);
    compiler_fence();
    if constexpr (kAppend) {
      if (fresh_p >= 0) fresh_page(stage_s[cstage], np == 2, fresh_p);
    }
    compiler_fence();
    process_pair(stage_s[cstage], np == 2, pos0);
    if (++cstage == kStages) cstage = 0;
    compiler_fence();
    ++consumed;
  };
  p_seek();
#pragma unroll
  for (int s = 0; s < kStages; ++s) produce();
  Cursor cons = start;
  while (cons.u < u1) {
    begin_segment(cons);
    // the segment's units in the range: its pages as pairs (a single page
    // last when their count is odd), then its tail if the range reaches it
    const int unit_end = min(cons.nunits, cons.unit + (u1 - cons.u));
    const int page_end = min(unit_end, cons.full);
    int unit = cons.unit;
    while (unit < page_end) {
      const int np = (unit + 1 < page_end) ? 2 : 1;
      // kAppend: with no tail, the segment's last page holds the new token
      const int fresh_p = (kAppend && cons.tail == 0 && unit + np == cons.full) ? cons.full - 1 : -1;
      consume_pair(np, unit * kPage, fresh_p);
      unit += np;
    }
    if (unit_end > cons.full) process_tail(cons.tail, cons.full * kPage);
    end_segment();
    advance(cons, unit_end - cons.unit);
  }
  if constexpr (kPacked) store_kept();
}

// Merge, for (sequence b, KV head h), the partial results of the waves whose
// unit ranges touched (b, h) (recorded by the wave owning its first unit): m in
// log2 units, O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s with M the
// max over the slots s. A block serves hb heads of one (b, h): hb x R slot
// groups x 32 / QW threads, each thread 4 * QW consecutive outputs. Thread
// group r merges slots r, r + R, ... online (one slot each when R covers them,
// as the launch sizes it); the groups' maxima meet in LDS, each group rescales
// to the common maximum, and the R groups add up in a fixed binary tree (same
// order every call). QW only changes which thread computes an output, not how:
// results are the same for every QW.
// With cu_q (several query tokens per sequence) blockIdx.y is a virtual
// sequence, column tile bv % ct_n of sequence bv / ct_n (see tile_span), and
// the G columns of a slot are (token, head) pairs, column jj = token
// tile * tpt + jj / gq, head jj % gq; columns past the sequence's token count
// are merged but not stored.
constexpr int kReduceThreads = 1024;
template <int QW>
__global__ __launch_bounds__(kReduceThreads) void splitk_reduce_kernel(
    const float* __restrict__ slots, const int32_t* __restrict__ total_units,
    const int2* __restrict__ seg_waves, const int32_t* __restrict__ ctx_lens, int32_t max_pages,
    int32_t hkv, int32_t G, int32_t W, __half* __restrict__ out, const int32_t* __restrict__ cu_q,
    int32_t gq, int32_t total_q, int32_t hb, int32_t R, int32_t ct_n, int32_t tpt) {
  constexpr int kLanes = 32 / QW;  // threads per (head, slot group)
  // a block has at most kReduceThreads / QW threads (the launch sizes it so)
  __shared__ float red_m[32], red_l[32];
  __shared__ f4 red_o[kReduceThreads];
  const int groups = (G + hb - 1) / hb;
  const int h = blockIdx.x / groups, b = blockIdx.y;
  const int t = threadIdx.x, nt = blockDim.x;
  const int q = t % kLanes, rg = t / kLanes;  // output block; (head, slot group) index
  const int r = rg % R, jb = rg / R;
  const int jj = (blockIdx.x % groups) * hb + jb;
  const int d0 = 4 * QW * q;
  const bool live = jj < G;
  __half* o = nullptr;
  bool store = live;
  int n = 0;
  if (cu_q != nullptr) {
    const int bs = b / ct_n;
    const int q0 = cu_q[bs], tq = (b - bs * ct_n) * tpt + (live ? jj : 0) / gq;
    // rows outside [0, total_q) are never written, whatever cu_q holds
    store = live && tq < cu_q[bs + 1] - q0 && q0 >= 0 && (int64_t)q0 + tq < total_q;
    o = out + (((int64_t)q0 + tq) * hkv * gq + h * gq + jj % gq) * kHeadDim + d0;
    const VSpan v = tile_span(b, ctx_lens, max_pages, cu_q, ct_n, tpt);
    n = v.full + (v.tail ? 1 : 0);
  } else {
    n = units_of(ctx_lens[b], max_pages);
    o = out + ((int64_t)b * hkv * G + h * G + jj) * kHeadDim + d0;
  }
  const int64_t bh = (int64_t)b * hkv + h;
  const int64_t U = total_units[0];
  if (n <= 0 || U <= 0) {
    if (r == 0 && store)
      for (int i = 0; i < QW; ++i) *reinterpret_cast<uint2*>(o + 4 * i) = make_uint2(0u, 0u);
    return;
  }
  const int2 ws = seg_waves[bh];
  float M = kNegInf, L = 0.f;
  f4 acc[QW];
  for (int i = 0; i < QW; ++i) acc[i] = f4{0.f, 0.f, 0.f, 0.f};
  auto join = [&](int wv) {
    const float* sl = slots + ((bh + wv) * G + jj) * kSlotStride;
    const float ms = sl[kHeadDim], ls = sl[kHeadDim + 1];
    f4 os[QW];
    for (int i = 0; i < QW; ++i) os[i] = *reinterpret_cast<const f4*>(sl + d0 + 4 * i);
    if (ms == kNegInf) return;
    const float Mn = fmaxf(M, ms);
    const float a = (M == kNegInf) ? 0.f : exp2f(M - Mn);
    const float c = exp2f(ms - Mn);
    // one rounding order for every QW: each term is fma(old, a, new * c)
    L = fmaf(L, a, ls * c);
    for (int i = 0; i < QW; ++i)
      for (int k = 0; k < 4; ++k) acc[i][k] = fmaf(acc[i][k], a, os[i][k] * c);
    M = Mn;
  };
  if (live) {
    if (U >= W) {
      // every range holds at least one unit: the waves ws.x .. ws.y
      for (int wv = ws.x + r; wv <= ws.y; wv += R) join(wv);
    } else {
      // every range holds at most one unit, so the (b, h)'s n units sit in
      // n waves, the owners of its units (the first one's range is that unit)
      const int64_t first = (int64_t)ws.x * U / W;
      for (int k = r; k < n; k += R) join(owner_wave(first + k, U, W));
    }
  }
  if (R > 1) {
    if (q == 0) red_m[rg] = M;
    __syncthreads();
    float Mh = kNegInf;
    for (int k = 0; k < R; ++k) Mh = fmaxf(Mh, red_m[jb * R + k]);
    const float a = (M == kNegInf) ? 0.f : exp2f(M - Mh);
    for (int i = 0; i < QW; ++i) {
      for (int k = 0; k < 4; ++k) acc[i][k] = __fmul_rn(acc[i][k], a);  // not fused into the adds below
      red_o[i * nt + t] = acc[i];
    }
    L = __fmul_rn(L, a);
    if (q == 0) red_l[rg] = L;
    __syncthreads();
    for (int stride = R / 2; stride > 0; stride /= 2) {
      if (r < stride) {
        for (int i = 0; i < QW; ++i) {
          acc[i] += red_o[i * nt + t + kLanes * stride];
          red_o[i * nt + t] = acc[i];
        }
        if (q == 0) {
          L += red_l[rg + stride];
          red_l[rg] = L;
        }
      }
      __syncthreads();
    }
    L = red_l[jb * R];
  }
  if (r != 0 || !store) return;
  const float inv = 1.0f / L;
  for (int i = 0; i < QW; ++i) {
    __half2 lo = __floats2half2_rn(acc[i][0] * inv, acc[i][1] * inv);
    __half2 hi = __floats2half2_rn(acc[i][2] * inv, acc[i][3] * inv);
    uint2 pk;
    pk.x = *reinterpret_cast<uint32_t*>(&lo);
    pk.y = *reinterpret_cast<uint32_t*>(&hi);
    *reinterpret_cast<uint2*>(o + 4 * i) = pk;
  }
}

// pages and tails are written only by the kAppend instantiations, whose
// callers pass writable buffers
template <int G, bool kMQ, int kBits, bool kAppend>
hipError_t launch_g(const s4kv_shape& s, int W, const void* q, const void* pages,
                    const void* tail_k, const void* tail_v, const int32_t* block_table,
                    const int32_t* ctx_lens, int32_t* total_units, int2* seg_waves, float sm_scale,
                    float* slots, const int32_t* cu_q, int32_t gq, int32_t total_q,
                    const void* k_new, const void* v_new, hipStream_t stream, int32_t ct_n,
                    int32_t tpt) {
  hipLaunchKernelGGL((decode_stream_kernel<G, kMQ, kBits, kAppend>), dim3(W), dim3(64), 0, stream,
                     static_cast<const __half*>(q), static_cast<uint8_t*>(const_cast<void*>(pages)),
                     static_cast<__half*>(const_cast<void*>(tail_k)),
                     static_cast<__half*>(const_cast<void*>(tail_v)),
                     block_table, ctx_lens, total_units, seg_waves, s.num_seqs, s.max_pages_per_seq,
                     s.num_kv_heads, sm_scale, slots, cu_q, gq, total_q,
                     static_cast<const __half*>(k_new), static_cast<const __half*>(v_new), ct_n,
                     tpt);
  return hipGetLastError();
}

// one instantiation per column count 1..16
template <bool kMQ, int kBits, bool kAppend = false>
hipError_t launch_columns(int G, const s4kv_shape& s, int W, const void* q, const void* pages,
                          const void* tail_k, const void* tail_v, const int32_t* block_table,
                          const int32_t* ctx_lens, int32_t* total_units, int2* seg_waves,
                          float sm_scale, float* slots, const int32_t* cu_q, int32_t gq,
                          int32_t total_q, hipStream_t stream, const void* k_new = nullptr,
                          const void* v_new = nullptr, int32_t ct_n = 1, int32_t tpt = 1) {
  switch (G) {
#define S4KV_CASE(g)                                                                             \
  case g:                                                                                        \
    return launch_g<g, kMQ, kBits, kAppend>(s, W, q, pages, tail_k, tail_v, block_table,         \
                                            ctx_lens, total_units, seg_waves, sm_scale, slots,  \
                                            cu_q, gq, total_q, k_new, v_new, stream, ct_n, tpt);
    S4KV_CASE(1) S4KV_CASE(2) S4KV_CASE(3) S4KV_CASE(4) S4KV_CASE(5) S4KV_CASE(6) S4KV_CASE(7)
    S4KV_CASE(8) S4KV_CASE(9) S4KV_CASE(10) S4KV_CASE(11) S4KV_CASE(12) S4KV_CASE(13)
    S4KV_CASE(14) S4KV_CASE(15) S4KV_CASE(16)
#undef S4KV_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int resident_waves() {
  // one wave per work-group, two per SIMD, four SIMDs per CU; the first call
  // sizes it (a function-local static: its initialization is thread-safe)
  static const int cached = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    return cus * 8 > kMaxWaves ? kMaxWaves : cus * 8;
  }();
  return cached;
}

namespace {
// Grid of a decode stream launch whose kernel runs per_simd waves per SIMD
// (resident_waves() counts two); the workspace holds slots for kMaxWaves.
int stream_waves(int per_simd) { return std::min(resident_waves() / 2 * per_simd, kMaxWaves); }
}  // namespace

// Workspace: [total units, padded to 256 B] [first / last wave per (b, h),
// padded to 256 B] [partial slots].
namespace {
constexpr size_t kHeaderBytes = 256;
size_t seg_bytes(const s4kv_shape& s) {
  return ((size_t)s.num_seqs * s.num_kv_heads * sizeof(int2) + 255) & ~size_t(255);
}
}  // namespace

SplitWorkspace split_workspace(const s4kv_shape& s, void* workspace) {
  char* ws = static_cast<char*>(workspace);
  SplitWorkspace w;
  w.total_units = reinterpret_cast<int32_t*>(ws);
  w.seg_waves = reinterpret_cast<int32_t*>(ws + kHeaderBytes);
  w.slots = reinterpret_cast<float*>(ws + kHeaderBytes + seg_bytes(s));
  return w;
}

namespace {
hipError_t launch_merge(const s4kv_shape& s, int W, int32_t max_ctx, const SplitWorkspace& ws,
                        const int32_t* ctx_lens, void* out, int G, const int32_t* cu_q, int32_t gq,
                        int32_t total_q, hipStream_t stream, int32_t ct_n = 1, int32_t tpt = 1) {
  // Slot groups per (sequence, head): the number of waves that share a (b, h)
  // when every context is max_ctx long (W waves over B * Hkv * pages units),
  // rounded up to a power of two, at most 32. Heads per block: as many as fit
  // 1024 threads next to the R groups. This only sizes the launch; any count
  // of sharing waves is merged correctly.
  const int64_t per_bh = ((int64_t)max_ctx + kPage - 1) / kPage;
  const int64_t units = (int64_t)s.num_seqs * s.num_kv_heads * per_bh;
  const int64_t share = ((int64_t)W * per_bh + units - 1) / (units > 0 ? units : 1);
  int R = 1;
  while (R < share && R < 32) R *= 2;
  const int hb = std::max(1, std::min(G, kReduceThreads / (32 * R)));
  const int groups = (G + hb - 1) / hb;
  // Outputs per thread: 4, or 8 / 16 when four per thread would need more
  // waves than the GPU holds at once (a merge of many columns or virtual
  // sequences then runs in one or a few rounds of resident waves, each thread
  // with several loads in flight, rather than in many rounds of one-load waves).
  const int64_t threads = (int64_t)s.num_seqs * s.num_kv_heads * groups * 32 * R * hb;
  const int64_t resident = (int64_t)resident_waves() * 4 * 64;  // 32 waves per CU
  const int QW = threads <= resident ? 1 : threads <= 2 * resident ? 2 : 4;
  const dim3 grid(s.num_kv_heads * groups, s.num_seqs), block(32 / QW * R * hb);
  const int2* segs = reinterpret_cast<const int2*>(ws.seg_waves);
  __half* o = static_cast<__half*>(out);
  if (QW == 1)
    hipLaunchKernelGGL(splitk_reduce_kernel<1>, grid, block, 0, stream, ws.slots, ws.total_units,
                       segs, ctx_lens, s.max_pages_per_seq, s.num_kv_heads, G, W, o, cu_q, gq,
                       total_q, hb, R, ct_n, tpt);
  else if (QW == 2)
    hipLaunchKernelGGL(splitk_reduce_kernel<2>, grid, block, 0, stream, ws.slots, ws.total_units,
                       segs, ctx_lens, s.max_pages_per_seq, s.num_kv_heads, G, W, o, cu_q, gq,
                       total_q, hb, R, ct_n, tpt);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<4>, grid, block, 0, stream, ws.slots, ws.total_units,
                       segs, ctx_lens, s.max_pages_per_seq, s.num_kv_heads, G, W, o, cu_q, gq,
                       total_q, hb, R, ct_n, tpt);
  return hipGetLastError();
}
size_t workspace_for_columns(const s4kv_shape& s, int columns) {
  const size_t nslots = (size_t)s.num_seqs * s.num_kv_heads + kMaxWaves;
  return kHeaderBytes + seg_bytes(s) + nslots * columns * kSlotStride * sizeof(float);
}
}  // namespace

hipError_t launch_split_merge(const s4kv_shape& s, int W, int32_t max_ctx, const SplitWorkspace& ws,
                              const int32_t* ctx_lens, void* out, hipStream_t stream) {
  const int G = s.num_q_heads / s.num_kv_heads;
  return launch_merge(s, W, max_ctx, ws, ctx_lens, out, G, nullptr, G, s.num_seqs, stream);
}

size_t workspace_bytes(const s4kv_shape& s) {
  return workspace_for_columns(s, s.num_q_heads / s.num_kv_heads);
}

size_t mq_workspace_bytes(const s4kv_shape& s, int32_t max_q) {
  const MqTiling t = mq_tiling(s, max_q);
  s4kv_shape sv = s;
  sv.num_seqs = static_cast<int32_t>(t.virtual_seqs);
  return workspace_for_columns(sv, t.columns);
}

hipError_t launch_paged_decode(const s4kv_shape& s, const void* q, const void* pages,
                               const void* tail_k, const void* tail_v,
                               const int32_t* block_table, const int32_t* ctx_lens,
                               int32_t max_ctx, float sm_scale, void* out, void* workspace,
                               hipStream_t stream, int bits) {
  const SplitWorkspace ws = split_workspace(s, workspace);
  const int G = s.num_q_heads / s.num_kv_heads;
  const int W = stream_waves(waves_per_simd(G, false, bits));
  const hipError_t e =
      (bits == 2)
          ? launch_columns<false, 2>(G, s, W, q, pages, tail_k, tail_v, block_table, ctx_lens,
                                     ws.total_units, reinterpret_cast<int2*>(ws.seg_waves), sm_scale,
                                     ws.slots, nullptr, G, s.num_seqs, stream)
          : launch_columns<false, 4>(G, s, W, q, pages, tail_k, tail_v, block_table, ctx_lens,
                                     ws.total_units, reinterpret_cast<int2*>(ws.seg_waves), sm_scale,
                                     ws.slots, nullptr, G, s.num_seqs, stream);
  if (e != hipSuccess) return e;
  return launch_split_merge(s, W, max_ctx, ws, ctx_lens, out, stream);
}

hipError_t launch_paged_decode_append(const s4kv_shape& s, const void* q, const void* k_new,
                                      const void* v_new, void* pages, void* tail_k, void* tail_v,
                                      const int32_t* block_table, const int32_t* ctx_lens,
                                      int32_t max_ctx, float sm_scale, void* out, void* workspace,
                                      hipStream_t stream) {
  const SplitWorkspace ws = split_workspace(s, workspace);
  const int W = resident_waves();
  const int G = s.num_q_heads / s.num_kv_heads;
  const hipError_t e = launch_columns<false, 4, true>(
      G, s, W, q, pages, tail_k, tail_v, block_table, ctx_lens, ws.total_units,
      reinterpret_cast<int2*>(ws.seg_waves), sm_scale, ws.slots, nullptr, G, s.num_seqs, stream,
      k_new, v_new);
  if (e != hipSuccess) return e;
  return launch_split_merge(s, W, max_ctx, ws, ctx_lens, out, stream);
}

hipError_t launch_paged_mq(const s4kv_shape& s, const void* q, const int32_t* cu_q, int32_t max_q,
                           int32_t total_q, const void* pages, const void* tail_k, const void* tail_v,
                           const int32_t* block_table, const int32_t* ctx_lens, int32_t max_ctx,
                           float sm_scale, void* out, void* workspace, hipStream_t stream) {
  // the stream and the merge run over virtual sequences, one per column tile
  const MqTiling t = mq_tiling(s, max_q);
  s4kv_shape sv = s;
  sv.num_seqs = static_cast<int32_t>(t.virtual_seqs);
  const SplitWorkspace ws = split_workspace(sv, workspace);
  const int W = stream_waves(waves_per_simd(t.columns, true, 4));
  const int gq = s.num_q_heads / s.num_kv_heads;
  const hipError_t e = launch_columns<true, 4>(
      t.columns, sv, W, q, pages, tail_k, tail_v, block_table, ctx_lens, ws.total_units,
      reinterpret_cast<int2*>(ws.seg_waves), sm_scale, ws.slots, cu_q, gq, total_q, stream,
      nullptr, nullptr, t.ct_n, t.tpt);
  if (e != hipSuccess) return e;
  return launch_merge(sv, W, max_ctx, ws, ctx_lens, out, t.columns, cu_q, gq, total_q, stream,
                      t.ct_n, t.tpt);
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  if (g_scratch_ptr[dev] == nullptr) return hipErrorInvalidSymbol;
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_paged_decode_append_noalloc(const s4kv_shape& s, const void* q, const void* k_new,
                                              const void* v_new, void* pages, void* tail_k,
                                              void* tail_v, const int32_t* block_table,
                                              const int32_t* ctx_lens, int32_t max_ctx,
                                              float sm_scale, void* out, hipStream_t stream) {
  void* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_paged_decode_append(s, q, k_new, v_new, pages, tail_k, tail_v, block_table,
                                    ctx_lens, max_ctx, sm_scale, out, ws, stream);
}

}  // namespace s4kv
