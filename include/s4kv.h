/*
 * s4kv -- int4 KIVI paged KV cache for AMD Instinct MI355X (gfx950).
 *
 * The method: the S4 KV product page ("int4 KV-Cache-Kompression fuer vLLM",
 * header paragraph and "Funktionsweise" step 1) stores the paged-attention KV
 * cache in int4 instead of fp16, KIVI style and asymmetric: KEY quantized per
 * channel, VALUE per token; supported models have head_dim 128 and standard
 * attention, and anything else is refused up front ("fail-fast", sections
 * "Highlights" and "FAQ"). Pages of 16 tokens reached through a page table
 * follow the PagedAttention explainers (gyaansetu.com "KV-Cache und
 * PagedAttention", section "Wie PagedAttention das loest").
 *
 * This library implements
 *   - s4kv_quantize_append: append new K/V tokens of each sequence; a page is
 *     quantized to int4 when its 16th token arrives, earlier tokens of the
 *     page wait in an fp16 residual tail;
 *   - s4kv_paged_decode: one decode step of attention for every sequence over
 *     its int4 pages plus its fp16 tail (GQA, split over pages, cross-split
 *     softmax reduction);
 *   - s4kv_paged_decode_append: the two above for one new token per
 *     sequence, fused into the decode's launch (bit-identical results);
 *   - s4kv_fp16_append / s4kv_fp16_paged_decode: the same over an fp16 paged
 *     cache, the control path the int4 cache is measured against.
 *
 * Quantizer (per group of fp16 values x): zero z = min(x) as fp16, scale
 * s = fp16((max - min) / 15) computed in fp32, code = clamp(rint_even((x - z)
 * / s), 0, 15) in IEEE fp32 with the stored fp16 s and z, codes 0 and scale
 * +0 when s is 0, -0 stored as +0. Dequantized value: code * s + z.
 *
 * Conventions for every call:
 *   - Pointers named "device" are HIP device pointers; the caller allocates
 *     and owns all memory, including the decode workspace. The library never
 *     allocates, holds no state between calls, and is safe to call from
 *     several host threads.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; no call synchronizes the host.
 *   - Shapes are checked on the host before anything is launched; a bad shape
 *     or argument returns an error status and enqueues nothing. Device-side
 *     preconditions (listed per call) are not checked in the kernels.
 *
 * Page format (one "chunk" per physical page and KV head; the pool is
 * uint8 pages[num_pages][num_kv_heads][S4KV_CHUNK_STRIDE]):
 *   offset    0: K codes, 1024 B      offset 1024: V codes, 1024 B
 *   offset 2048: K scale fp16[128]    offset 2304: K zero fp16[128]   (per channel)
 *   offset 2560: V scale fp16[16]     offset 2592: V zero fp16[16]    (per token)
 *   offset 2624: 64 B padding (written as zero)
 * Codes are 4-bit, two per byte, low nibble first. Inside the 1024-B K block,
 * byte 16*l + 4*m + k/2 (nibble k = 0..7 of dword m = 0..3 of 16-byte lane
 * block l = 16*g + t) holds the K code of token t, channel
 * d = 32*m + 8*g + 2*(k%4) + k/4. Inside the V block, lane block
 * l = 16*g + r, dword m, nibble k holds the V code of token
 * t = 4*g + 2*(k%2) + k/4, channel d = 16*(2*m + (k%4)/2) + r.
 * (This order lets the decode kernel feed each 16-byte load straight into
 * matrix-core operands.)
 */
#ifndef S4KV_H_
#define S4KV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define S4KV_HEAD_DIM 128
#define S4KV_PAGE_SIZE 16
#define S4KV_CHUNK_BYTES 2624 /* bytes of a chunk that carry data */
#define S4KV_CHUNK_STRIDE 2688 /* chunk stride in the pool (128-byte multiple) */
#define S4KV_MAX_GROUP 16 /* largest supported query heads per KV head */

typedef enum s4kv_status {
  S4KV_OK = 0,
  S4KV_ERR_INVALID_ARG = 1, /* null pointer, negative or zero count, bad bound */
  S4KV_ERR_UNSUPPORTED = 2, /* head_dim != 128, page_size != 16, Hq % Hkv != 0,
                               Hq / Hkv > 16: the model is refused */
  S4KV_ERR_WORKSPACE = 3,   /* decode workspace smaller than required */
  S4KV_ERR_HIP = 4,         /* a HIP launch failed (hipGetLastError) */
  S4KV_ERR_SCRATCH_LIMIT = 5 /* s4kv_paged_decode_append_noalloc: the shape needs more
                               decode workspace than S4KV_NOALLOC_SCRATCH_BYTES */
} s4kv_status;

typedef struct s4kv_shape {
  int32_t num_seqs;          /* B: sequences in the batch (rows of block table) */
  int32_t num_q_heads;       /* Hq */
  int32_t num_kv_heads;      /* Hkv; Hq must be a multiple, Hq / Hkv <= 16 */
  int32_t head_dim;          /* must be 128 */
  int32_t page_size;         /* must be 16 */
  int32_t num_pages;         /* physical pages in this layer's pool */
  int32_t max_pages_per_seq; /* row length of the block table */
} s4kv_shape;

/* Check a shape without touching the GPU (S4 KV page, "FAQ": unsupported
 * models are refused at start instead of producing wrong output).
 * Returns S4KV_OK, S4KV_ERR_INVALID_ARG (null, counts < 1) or
 * S4KV_ERR_UNSUPPORTED. */
s4kv_status s4kv_validate(const s4kv_shape* shape);

/* Human-readable name of a status. Never NULL; static storage. */
const char* s4kv_status_string(s4kv_status status);

/* Bytes the caller must allocate for one layer's page pool:
 * num_pages * num_kv_heads * S4KV_CHUNK_STRIDE. 0 if the shape is invalid. */
size_t s4kv_pool_bytes(const s4kv_shape* shape);

/* Bytes of ONE fp16 residual-tail buffer (K or V) for one layer:
 * num_seqs * num_kv_heads * 16 * 128 * 2, layout fp16 [B][Hkv][16][128]
 * indexed by the token's position modulo 16. 0 if the shape is invalid. */
size_t s4kv_tail_bytes(const s4kv_shape* shape);

/* Append new tokens to every sequence of one layer.
 *
 * Args (device pointers unless noted):
 *   k, v         fp16 [total_new][Hkv][128], contiguous; the new tokens of
 *                sequence b are rows cu_new[b] .. cu_new[b+1]-1, in order.
 *   cu_new       int32 [B+1], cu_new[0] = 0, non-decreasing.
 *   slot         int32 [B]: tokens already cached for sequence b, i.e. the
 *                position of its first new token.
 *   max_new      host int: an upper bound on cu_new[b+1]-cu_new[b] for every
 *                b (1 for a decode step). It sizes the launch only.
 *   block_table  int32 [B][max_pages_per_seq]: physical page of each logical
 *                page of each sequence.
 *   pages        the layer's pool (s4kv_pool_bytes); written.
 *   tail_k/v     the layer's fp16 tails (s4kv_tail_bytes each); read and written.
 * Effect: for every page that becomes full, its 16 tokens (older ones from
 * the tail, new ones from k/v) are quantized and written to the chunk
 * block_table[b][page] of each KV head; new tokens of a page that stays
 * partial are written to the tail at (position % 16).
 * Device preconditions: new tokens per sequence <= max_new; slot[b] + new
 * tokens <= 16 * max_pages_per_seq; block ids in [0, num_pages); the tail of
 * b holds its tokens 16*floor(slot/16) .. slot-1 (as left by earlier calls);
 * no two sequences write the same physical page in one call; k and v finite.
 * Returns S4KV_OK or an error before any launch; S4KV_ERR_HIP if the launch
 * fails. */
s4kv_status s4kv_quantize_append(const s4kv_shape* shape, const void* k, const void* v,
                                 const int32_t* cu_new, const int32_t* slot, int32_t max_new,
                                 const int32_t* block_table, void* pages, void* tail_k,
                                 void* tail_v, void* stream);

/* Bytes of device workspace s4kv_paged_decode needs for this shape and a
 * context bound max_ctx (host int). 0 if the shape is invalid or max_ctx < 1. */
size_t s4kv_decode_workspace_bytes(const s4kv_shape* shape, int32_t max_ctx);

/* One decode step of attention for every sequence of one layer.
 *
 * For sequence b and query head j (KV head h = j / (Hq/Hkv)):
 *   O[b][j] = sum_t softmax_t(sm_scale * q[b][j] . k_t) v_t over the ctx_lens[b]
 * cached tokens, where k_t, v_t are the dequantized int4 values for tokens in
 * full pages and the fp16 tail values for the last ctx_lens[b] % 16 tokens.
 *
 * Args (device pointers unless noted):
 *   q            fp16 [B][Hq][128].
 *   pages, tail_k, tail_v  the layer's cache (read only).
 *   block_table  int32 [B][max_pages_per_seq].
 *   ctx_lens     int32 [B]: cached tokens per sequence (after any append).
 *   max_ctx      host int >= every ctx_lens[b]; sizes the launch and workspace.
 *   sm_scale     host float, logit scale (1/sqrt(128) for standard attention).
 *   out          fp16 [B][Hq][128]; written.
 *   workspace    device scratch of at least s4kv_decode_workspace_bytes
 *                (caller-owned; contents on entry do not matter).
 * Device preconditions: 1 <= ctx_lens[b] <= max_ctx and <= 16 *
 * max_pages_per_seq; block ids of full pages in [0, num_pages). A sequence
 * with ctx_lens[b] <= 0 gets an all-zero output.
 * Returns S4KV_OK; S4KV_ERR_INVALID_ARG / S4KV_ERR_UNSUPPORTED /
 * S4KV_ERR_WORKSPACE before any launch; S4KV_ERR_HIP if a launch fails. */
s4kv_status s4kv_paged_decode(const s4kv_shape* shape, const void* q, const void* pages,
                              const void* tail_k, const void* tail_v,
                              const int32_t* block_table, const int32_t* ctx_lens,
                              int32_t max_ctx, float sm_scale, void* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* One decode step with its append fused in: s4kv_quantize_append of one new
 * token per sequence followed by s4kv_paged_decode, as one call (one launch
 * of the decode stream, then the split merge). The pages' method is the same
 * (S4 KV product page, "Funktionsweise" steps 1 and 2): the new token joins
 * the fp16 tail, or completes its page, which is then quantized by the rule
 * above; attention then covers every cached token including the new one.
 * Pages, tails and outputs are bit-identical to the two separate calls.
 *
 * Args (device pointers unless noted):
 *   q            fp16 [B][Hq][128].
 *   k_new, v_new fp16 [B][Hkv][128]: the new token of every sequence.
 *   pages, tail_k, tail_v  the layer's cache; updated in place.
 *   block_table  int32 [B][max_pages_per_seq]; must map the page that the
 *                new token lands in.
 *   ctx_lens     int32 [B]: cached tokens per sequence AFTER the append, so
 *                the new token sits at position ctx_lens[b] - 1 and the
 *                cache held ctx_lens[b] - 1 tokens on entry.
 *   max_ctx, sm_scale, out, workspace, workspace_bytes, stream: as for
 *                s4kv_paged_decode (same workspace size).
 * Device preconditions: those of s4kv_paged_decode. A sequence with
 * ctx_lens[b] <= 0 takes no token and gets an all-zero output. Calls that
 * share the cache buffers must not overlap.
 * Returns as s4kv_paged_decode. */
s4kv_status s4kv_paged_decode_append(const s4kv_shape* shape, const void* q, const void* k_new,
                                     const void* v_new, void* pages, void* tail_k, void* tail_v,
                                     const int32_t* block_table, const int32_t* ctx_lens,
                                     int32_t max_ctx, float sm_scale, void* out, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ---- allocation-free decode step ----
 *
 * For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The same call as s4kv_paged_decode_append (same arguments, same
 * kernels, bit-identical results) with the decode workspace taken from a
 * static array inside the library instead of an argument:
 *   - one array of S4KV_NOALLOC_SCRATCH_BYTES per device, created when the
 *     library's code is loaded on that device and held until the process
 *     ends; its address is looked up on the first call on a device;
 *   - a shape whose workspace (s4kv_decode_workspace_bytes) exceeds it is
 *     refused with S4KV_ERR_SCRATCH_LIMIT before anything is enqueued (the
 *     Llama-3.1-8B- and 70B-shaped decode steps need about 11 MB and 18 MB);
 *   - the call allocates nothing and frees nothing; every call on one device
 *     shares that device's array, and nothing in it needs to be cleared
 *     between calls (the call writes every workspace word it later reads),
 *     but calls that overlap on one device (different streams, or different
 *     host threads, without ordering between them) race on it and give
 *     undefined results;
 *   - the stream must belong to the current device.
 * Returns as s4kv_paged_decode_append, or S4KV_ERR_SCRATCH_LIMIT. */
#define S4KV_NOALLOC_SCRATCH_BYTES (32u << 20)
s4kv_status s4kv_paged_decode_append_noalloc(const s4kv_shape* shape, const void* q,
                                             const void* k_new, const void* v_new, void* pages,
                                             void* tail_k, void* tail_v,
                                             const int32_t* block_table, const int32_t* ctx_lens,
                                             int32_t max_ctx, float sm_scale, void* out,
                                             void* stream);

/* ---- 2-bit KIVI pages ----
 *
 * The same cache with 2-bit codes: the KIVI paper the KV-cache explainer
 * cites (analyticslegends.ai, "Quellen", entry 17) quantizes the cache
 * asymmetrically to 2 bits, KEY per channel and VALUE per token. Same
 * grouping, tail, rounding rule and entry-point conventions as the int4
 * calls, with scale = (max - min) / 3 and codes 0..3.
 *
 * 2-bit page format: pool uint8 [num_pages][num_kv_heads][1664]; each chunk
 * holds 1600 bytes of data, then 64 bytes of padding (written as zero):
 *   [   0, 512) K codes   [ 512,1024) V codes
 *   [1024,1280) K scale fp16[128] (per channel)   [1280,1536) K zero fp16[128]
 *   [1536,1568) V scale fp16[16] (per token)      [1568,1600) V zero fp16[16]
 * Code blocks: lane L = 16 g + c owns bytes 8 L .. 8 L + 7, two little-endian
 * 32-bit words dd = 0, 1, each code 2 bits wide:
 *   K (token c): word dd holds channel 32 m + 8 g + i for m = 2 dd + mm
 *     (mm = 0, 1) and i = 0..7, at bit 8 mm + 2 (i >> 1) + 16 (i & 1);
 *   V (channel offset c): word dd holds channel 16 (4 dd + s) + c of token
 *     4 g + k for s = 0..3 and k = 0..3, at bit 4 s + 2 (k >> 1) + 16 (k & 1).
 * Full pages cost 100 bytes per token per KV head (5.12x denser than fp16). */
#define S4KV_K2_CHUNK_BYTES 1600  /* data bytes of one (page, KV head) chunk */
#define S4KV_K2_CHUNK_STRIDE 1664 /* chunk pitch in the pool (13 x 128 B) */

/* Bytes of one layer's 2-bit pool: num_pages * num_kv_heads * 1664; 0 if the
 * shape is invalid. The tails and the decode workspace are the int4 ones
 * (s4kv_tail_bytes, s4kv_decode_workspace_bytes). */
size_t s4kv_kivi2_pool_bytes(const s4kv_shape* shape);

/* s4kv_quantize_append with 2-bit codes: same arguments, statuses and device
 * preconditions; pages is the 2-bit pool. */
s4kv_status s4kv_kivi2_quantize_append(const s4kv_shape* shape, const void* k, const void* v,
                                       const int32_t* cu_new, const int32_t* slot,
                                       int32_t max_new, const int32_t* block_table, void* pages,
                                       void* tail_k, void* tail_v, void* stream);

/* s4kv_paged_decode over 2-bit pages: same arguments, statuses, workspace and
 * device preconditions; k_t, v_t of full pages are code * scale + zero of the
 * 2-bit codes. */
s4kv_status s4kv_kivi2_paged_decode(const s4kv_shape* shape, const void* q, const void* pages,
                                    const void* tail_k, const void* tail_v,
                                    const int32_t* block_table, const int32_t* ctx_lens,
                                    int32_t max_ctx, float sm_scale, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ---- multi-query attention over the int4 cache ----
 *
 * Several new query tokens per sequence attend over the same pages and tail:
 * the speculative-decoding verify step and small prefill chunks, the prefill
 * side of the two inference phases (polaris7.io signal page, "Verwandte
 * Marktsignale & Trends", the entry on KV caching, which names the prefill
 * and decoding phases). The new tokens' K and V are appended first
 * (s4kv_quantize_append), so ctx_lens counts them; token t of the T_b new
 * tokens of sequence b sits at cache position p = ctx_lens[b] - T_b + t and
 * attends causally:
 *   O[row][j] = sum_{s <= p} softmax_s(sm_scale * q[row][j] . k_s) v_s,
 *   row = cu_q[b] + t, KV head of j = j / (Hq/Hkv).
 * One launch serves every sequence. The (token, query head) pairs of a KV
 * head feed the matrix cores as columns, 16 at a time: with max_q * Hq / Hkv
 * <= 16 (speculative verify) one pass over the pages serves all of a
 * sequence's tokens; with more (a prefill chunk) the tokens are cut into
 * tiles of floor(16 / (Hq / Hkv)) whole tokens, each tile streaming the
 * pages up to its last token's position. Limits: num_seqs * tiles <= 65535
 * and num_seqs * tiles * Hkv * (max_pages_per_seq + 1) < 2^31, tiles =
 * ceil(max_q / tile tokens). */

/* Bytes of device workspace s4kv_paged_attention_mq needs (0 if the shape is
 * invalid, max_ctx < 1, max_q < 1 or the tiles exceed the limits above). */
size_t s4kv_mq_workspace_bytes(const s4kv_shape* shape, int32_t max_ctx, int32_t max_q);

/* Multi-query attention step.
 * Args (device pointers unless noted):
 *   q            fp16 [total_q][Hq][128]: the new tokens' queries, sequence by
 *                sequence.
 *   cu_q         int32 [B + 1]: sequence b's tokens are rows cu_q[b] ..
 *                cu_q[b + 1] - 1; cu_q[0] = 0, cu_q[B] = total_q.
 *   max_q        host int >= every T_b = cu_q[b + 1] - cu_q[b]; sizes the launch.
 *   total_q      host int, the number of query rows.
 *   pages, tail_k, tail_v, block_table, ctx_lens, max_ctx, sm_scale  as
 *                s4kv_paged_decode (ctx_lens includes the new tokens).
 *   out          fp16 [total_q][Hq][128]; written.
 *   workspace    device scratch of at least s4kv_mq_workspace_bytes.
 * Device preconditions: as s4kv_paged_decode, plus 1 <= T_b <= min(max_q,
 * ctx_lens[b]) and cu_q as above.
 * Returns S4KV_OK; S4KV_ERR_INVALID_ARG / S4KV_ERR_UNSUPPORTED (tiles beyond
 * the limits above) / S4KV_ERR_WORKSPACE before any launch; S4KV_ERR_HIP if a
 * launch fails. */
s4kv_status s4kv_paged_attention_mq(const s4kv_shape* shape, const void* q, const int32_t* cu_q,
                                    int32_t max_q, int32_t total_q, const void* pages,
                                    const void* tail_k, const void* tail_v,
                                    const int32_t* block_table, const int32_t* ctx_lens,
                                    int32_t max_ctx, float sm_scale, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ---- fp16 control path ----
 *
 * The same cache and decode step with K and V kept in fp16 (the format the
 * int4 cache replaces), for measuring the density / latency trade-off on the
 * same harness: the S4 KV product page ("FAQ", the question on inference
 * latency) says the int4 backend gives up some decode latency for density at
 * long contexts, and the KV-quantization guide on adechristanto.de (section
 * on separating weights, running state and reserved memory) notes that a
 * smaller KV element halves the payload term but not necessarily latency.
 *
 * fp16 page format (pool fp16 [num_pages][num_kv_heads][4096]): per (page, KV
 * head) the K block [16 tokens][128 channels], then the V block transposed,
 * [128 channels][16 tokens]. There is no separate tail: a sequence's last
 * page may be partial, and only its first ctx - 16 * (pages - 1) token slots
 * are defined. Same shape rules, statuses and conventions as above. */
#define S4KV_F16_CHUNK_BYTES 8192 /* bytes of one (page, KV head) fp16 chunk */

/* Bytes of one layer's fp16 pool: num_pages * num_kv_heads * 8192; 0 if the
 * shape is invalid. */
size_t s4kv_fp16_pool_bytes(const s4kv_shape* shape);

/* Append new K/V tokens to the fp16 pool of one layer.
 * Args as s4kv_quantize_append (k, v fp16 [total_new][Hkv][128]; cu_new,
 * slot, max_new, block_table); pages is the fp16 pool (written). Each new
 * token t of sequence b goes to slot t % 16 of page block_table[b][t / 16].
 * Device preconditions: as s4kv_quantize_append, without the tail ones.
 * Returns S4KV_OK, an argument / shape error before any launch, or
 * S4KV_ERR_HIP. */
s4kv_status s4kv_fp16_append(const s4kv_shape* shape, const void* k, const void* v,
                             const int32_t* cu_new, const int32_t* slot, int32_t max_new,
                             const int32_t* block_table, void* pages, void* stream);

/* One decode step over the fp16 pool: O[b][j] = sum_t softmax_t(sm_scale *
 * q[b][j] . k_t) v_t over the ctx_lens[b] cached tokens. Args and workspace
 * (s4kv_decode_workspace_bytes) as s4kv_paged_decode, without tails.
 * Device preconditions: 1 <= ctx_lens[b] <= max_ctx and <= 16 *
 * max_pages_per_seq; block ids of the ceil(ctx_lens[b] / 16) pages in
 * [0, num_pages). A sequence with ctx_lens[b] <= 0 gets an all-zero output.
 * Returns as s4kv_paged_decode. */
s4kv_status s4kv_fp16_paged_decode(const s4kv_shape* shape, const void* q, const void* pages,
                                   const int32_t* block_table, const int32_t* ctx_lens,
                                   int32_t max_ctx, float sm_scale, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ---- FP8 (E4M3) paged cache ----
 *
 * The quantized KV cache the KV-quantization guide on adechristanto.de
 * discusses most (sections on attention arithmetic in the quantized domain
 * and on default or calibrated scales): every K and V element is one FP8
 * byte, with scales of 1.0 by default or calibrated, per tensor or per
 * attention head. Here: OCP E4M3 (1 sign, 4 exponent bits of bias 7, 3
 * mantissa bits, largest finite 448, NaN = S.1111.111, no infinities) and one
 * fp32 scale per KV head for K and one for V (equal values give a per-tensor
 * scale). Queries stay fp16.
 *
 * Encode (append): y = fp16 input / scale as one IEEE fp32 division, then the
 * nearest E4M3 value, ties to even; |y| >= 448 saturates to +-448 (0x7E /
 * 0xFE); the sign is kept, also for a zero result. Decode: value(code) x scale.
 *
 * FP8 page format (pool uint8 [num_pages][num_kv_heads][4096]): per (page,
 * KV head) four 1024-byte blocks in matrix-core operand order. With L = 16 g +
 * c (g in 0..3, c in 0..15) and i in 0..15, byte 1024 j + 16 L + i holds
 *   j = 0, 1:  K[token c][channel 32 (2j + i/8) + 8g + i%8]
 *   j = 2, 3:  V[token 4g + i%4][channel 16 (4(j-2) + i/4) + c]
 * As in the fp16 pool there is no tail: a sequence's last page may be
 * partial, and only its first ctx - 16 * (pages - 1) token slots are defined.
 * Same shape rules, statuses and conventions as above. */
#define S4KV_FP8_CHUNK_BYTES 4096 /* bytes of one (page, KV head) FP8 chunk */

/* Bytes of one layer's FP8 pool: num_pages * num_kv_heads * 4096; 0 if the
 * shape is invalid. */
size_t s4kv_fp8_pool_bytes(const s4kv_shape* shape);

/* Quantize new K/V tokens to E4M3 and append them to the FP8 pool of one layer.
 * Args as s4kv_fp16_append, plus (device pointers):
 *   k_scale, v_scale  fp32 [num_kv_heads]: the scale of each KV head's K / V
 *                     (finite, > 0; the caller keeps them fixed for the
 *                     cache's lifetime, decode reads the same arrays).
 *   pages             the FP8 pool (written).
 * Each new token t of sequence b goes to slot t % 16 of page
 * block_table[b][t / 16], in the layout above.
 * Device preconditions: as s4kv_fp16_append.
 * Returns S4KV_OK, an argument / shape error before any launch, or
 * S4KV_ERR_HIP. */
s4kv_status s4kv_fp8_append(const s4kv_shape* shape, const void* k, const void* v,
                            const int32_t* cu_new, const int32_t* slot, int32_t max_new,
                            const int32_t* block_table, const float* k_scale,
                            const float* v_scale, void* pages, void* stream);

/* One decode step over the FP8 pool: O[b][j] = sum_t softmax_t(sm_scale *
 * q[b][j] . k_t) v_t over the ctx_lens[b] cached tokens, with k_t, v_t the
 * E4M3 values times k_scale[h] / v_scale[h] (h = j / (Hq/Hkv)). Args and
 * workspace (s4kv_decode_workspace_bytes) as s4kv_fp16_paged_decode, plus the
 * scale arrays of s4kv_fp8_append (device, read only).
 * Device preconditions: as s4kv_fp16_paged_decode.
 * Returns as s4kv_paged_decode. */
s4kv_status s4kv_fp8_paged_decode(const s4kv_shape* shape, const void* q, const void* pages,
                                  const int32_t* block_table, const int32_t* ctx_lens,
                                  int32_t max_ctx, float sm_scale, const float* k_scale,
                                  const float* v_scale, void* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* ---- Table checks (a debugging aid) ----
 *
 * The append and decode kernels trust the device preconditions stated above
 * for the block table and the context lengths (checking them in every page
 * step would cost the hot path). This call checks them on the device, on
 * demand, for callers that want to validate their tables before a call, in
 * a debug build of their own code or in tests. It reads block_table and
 * ctx_lens only within the shape's bounds and changes nothing else.
 *
 * For every sequence b it checks that 0 <= ctx_lens[b] <= 16 *
 * max_pages_per_seq (a negative length, which the calls treat as an empty
 * sequence, counts as a fault here) and, when max_ctx > 0, ctx_lens[b] <=
 * max_ctx; and for
 * every page p that holds one of the sequence's tokens, p < ceil(ctx_lens[b]
 * / 16) (the pages of its first min(ctx_lens[b], 16 * max_pages_per_seq)
 * tokens, the partial last page included, which an append completes), that
 * 0 <= block_table[b][p] < num_pages.
 *
 * Args (device pointers unless noted):
 *   block_table  int32 [B][max_pages_per_seq].
 *   ctx_lens     int32 [B].
 *   max_ctx      host int: the bound the next call will pass, or 0 to skip
 *                that comparison.
 *   report       int32 [4], written: [0] the sequences whose length is out of
 *                range; [1] the block-table entries in use that are out of
 *                range; [2] the smallest b with either fault, or -1; [3] that
 *                sequence's first out-of-range page, or -1 when only its
 *                length is out of range (or there is no fault).
 * One launch of one work-group; stream-ordered like every other call.
 * Returns S4KV_OK; S4KV_ERR_INVALID_ARG / S4KV_ERR_UNSUPPORTED before any
 * launch (null pointers, max_ctx < 0, invalid shape); S4KV_ERR_HIP if the
 * launch fails. */
s4kv_status s4kv_check_tables(const s4kv_shape* shape, const int32_t* block_table,
                              const int32_t* ctx_lens, int32_t max_ctx, int32_t* report,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* S4KV_H_ */
