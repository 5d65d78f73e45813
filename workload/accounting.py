"""Byte accounting for the KV cache (host arithmetic for reports; no kernels).

fp16 payload: the FP8 KV-cache capacity guide (adechristanto.de, section
"Gewichte, laufenden Zustand und reservierten Speicher trennen") gives the
unsharded KV payload as 2 x layers x KV heads x head_dim x held token
positions x bytes per element, and notes that scale metadata and block
rounding are not in it.

int4 KIVI layout (this library's page format): per full 16-token page and KV
head, K codes 16 x 128 nibbles (1024 B), V codes (1024 B), K scale and zero per
channel (2 x 128 fp16 = 512 B), V scale and zero per token (2 x 16 fp16 = 64 B):
2624 B, i.e. 164 B per token per KV head against 512 B in fp16. Tokens of the
not yet full page are fp16 (512 B per token per KV head).
"""

import numpy as np

PAGE = 16
HEAD_DIM = 128
CHUNK_BYTES = 2 * (PAGE * HEAD_DIM // 2) + 2 * 2 * HEAD_DIM + 2 * 2 * PAGE   # 2624
# 2-bit KIVI pages: codes 16 x 128 x 2 bits for K and V, same metadata
K2_CHUNK_BYTES = 2 * (PAGE * HEAD_DIM // 4) + 2 * 2 * HEAD_DIM + 2 * 2 * PAGE  # 1600
FP16_TOKEN_BYTES = 2 * HEAD_DIM * 2                                           # K + V, 512


def fp16_kv_bytes(layers, kv_heads, head_dim, tokens, bytes_per_elem=2):
    """2 x layers x KV heads x head_dim x tokens x bytes (fp16 payload)."""
    return 2 * layers * kv_heads * head_dim * tokens * bytes_per_elem


def int4_bytes_per_token_per_head():
    return CHUNK_BYTES / PAGE


def density_vs_fp16():
    return FP16_TOKEN_BYTES / int4_bytes_per_token_per_head()


def cache_bytes(ctx_lens, kv_heads, chunk_bytes=CHUNK_BYTES):
    """Bytes of the int4 cache (full pages) plus the fp16 tail, one layer,
    counting every sequence's pages (shared pages counted once per reader).
    chunk_bytes=K2_CHUNK_BYTES counts 2-bit pages."""
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    full = ctx // PAGE
    tail = ctx % PAGE
    return int(kv_heads * (full.sum() * chunk_bytes + tail.sum() * FP16_TOKEN_BYTES))


def decode_bytes(ctx_lens, num_q_heads, kv_heads, chunk_bytes=CHUNK_BYTES):
    """Algorithmic HBM bytes of one decode launch (one layer): the cache read
    (pages and tails), the block-table entries of the full pages, the context
    lengths, Q read and O written (fp16)."""
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    b = len(ctx)
    full = ctx // PAGE
    return int(cache_bytes(ctx, kv_heads, chunk_bytes) + 4 * full.sum() + 4 * b
               + 2 * (2 * b * num_q_heads * HEAD_DIM))


def append_step_bytes(ctx_lens, kv_heads):
    """Algorithmic bytes of appending one token to every sequence with
    ctx_lens[b] >= 1 (ctx_lens count the new token): its fp16 K/V read, then
    either its tail slot written or, when it completes a page, the page's 15
    earlier tail tokens read and the page's int4 chunk written."""
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    live = ctx > 0
    n = int(live.sum())
    done = int((live & (ctx % PAGE == 0)).sum())
    return int(kv_heads * (n * FP16_TOKEN_BYTES + (n - done) * FP16_TOKEN_BYTES
                           + done * ((PAGE - 1) * FP16_TOKEN_BYTES + CHUNK_BYTES)))


def fp16_decode_bytes(ctx_lens, num_q_heads, kv_heads):
    """Algorithmic HBM bytes of one fp16-cache decode launch (one layer): the
    fp16 K and V of every cached token, one block-table entry per page (full
    or partial), the context lengths, Q read and O written."""
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    b = len(ctx)
    pages = -(-ctx // PAGE)
    return int(kv_heads * ctx.sum() * FP16_TOKEN_BYTES + 4 * pages.sum() + 4 * b
               + 2 * (2 * b * num_q_heads * HEAD_DIM))


def mq_bytes(ctx_lens, t_counts, num_q_heads, kv_heads):
    """Algorithmic HBM bytes of one multi-query attention launch (one layer):
    the decode bytes with Q read and O written for every new token, plus the
    query-row offsets (B + 1 int32)."""
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    t = np.asarray(t_counts, dtype=np.int64)
    b = len(ctx)
    full = ctx // PAGE
    return int(cache_bytes(ctx, kv_heads) + 4 * full.sum() + 4 * b + 4 * (b + 1)
               + 2 * (2 * int(t.sum()) * num_q_heads * HEAD_DIM))


FP8_TOKEN_BYTES = 2 * HEAD_DIM                                                # K + V, 256


def fp8_decode_bytes(ctx_lens, num_q_heads, kv_heads):
    """Algorithmic HBM bytes of one FP8-cache decode launch (one layer): one
    byte per cached K and V element (the guide's payload with 1-byte
    elements), one block-table entry per page (full or partial), the context
    lengths, the K and V scale of each KV head, Q read and O written."""
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    b = len(ctx)
    pages = -(-ctx // PAGE)
    return int(kv_heads * ctx.sum() * FP8_TOKEN_BYTES + 4 * pages.sum() + 4 * b + 8 * kv_heads
               + 2 * (2 * b * num_q_heads * HEAD_DIM))


def quantize_bytes(n_tokens_flushed_pages, n_tail_tokens, kv_heads):
    """Algorithmic bytes of a bulk prefill quantize: fp16 K/V read for every
    token, int4 pages written for full pages, fp16 tail written."""
    pages = n_tokens_flushed_pages // PAGE
    return int(kv_heads * (n_tokens_flushed_pages * FP16_TOKEN_BYTES + pages * CHUNK_BYTES
                           + 2 * n_tail_tokens * FP16_TOKEN_BYTES))


def decode_bytes_unique(ctx_lens, num_q_heads, kv_heads, alias_pages, chunk_bytes=CHUNK_BYTES):
    """decode_bytes with every shared page counted once.

    ``alias_pages[b]``: how many of sequence b's first pages are shared pages
    (the sequences that share a prefix all alias its first pages, so the
    shared pages read by anyone are the first max(alias_pages) of them).
    decode_bytes counts a shared page once per sequence that reads it (logical
    bytes, what attention consumes); this counts each physical shared page
    once (unique bytes, what HBM must deliver when repeated reads of a page
    hit in a cache). Block-table entries stay counted per reader."""
    a = np.asarray(alias_pages, dtype=np.int64)
    dup = int(a.sum() - (a.max() if a.size else 0))
    return decode_bytes(ctx_lens, num_q_heads, kv_heads, chunk_bytes) - kv_heads * chunk_bytes * dup
