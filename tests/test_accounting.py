"""Byte accounting pinned to the figures the pages print (tests/golden/page_figures.json).

The fp16 payload formula is the one the FP8 KV-cache capacity guide gives
(adechristanto.de, section on separating weights, running state and reserved
memory); the int4 page size follows from the page format. Both feed the GB/s
that bench.py reports, so they are checked against the pages' own numbers.
"""

import json
import os

import numpy as np
import pytest

from workload import accounting as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")


def _figures():
    with open(GOLDEN) as f:
        return {g["name"]: g for g in json.load(f)["figures"]}


@pytest.mark.parametrize("name", ["fp16_kv_per_sequence_llama31_70b_4096",
                                  "fp16_kv_per_request_llama3_70b_32k",
                                  "fp16_kv_256_sequences_llama31_70b_4096"])
def test_fp16_payload_matches_printed_figures(name):
    g = _figures()[name]
    got = A.fp16_kv_bytes(g["layers"], g["kv_heads"], g["head_dim"], g["tokens"], g["bytes_per_elem"])
    assert g["lo"] <= got <= g["hi"], (name, got)


def test_int4_density_matches_printed_figure():
    g = _figures()["int4_kivi_density_vs_fp16"]
    d = A.density_vs_fp16()
    assert g["lo"] <= d <= g["hi"]
    # 164 B per token per KV head: codes 64 + 64, V scale/zero 4, K scale/zero 512 / 16
    assert A.int4_bytes_per_token_per_head() == 64 + 64 + 4 + 32
    assert A.CHUNK_BYTES == 2624


def test_cache_bytes_counts_pages_and_tail():
    # 37 tokens = 2 full pages + 5 tail tokens, per KV head
    assert A.cache_bytes([37], 3) == 3 * (2 * 2624 + 5 * 512)
    assert A.cache_bytes([16, 0, 15], 1) == 2624 + 15 * 512
    # decode bytes add block-table entries, ctx lengths, Q and O
    b = A.decode_bytes(np.array([37]), 12, 3)
    assert b == A.cache_bytes([37], 3) + 4 * 2 + 4 + 2 * (2 * 12 * 128)


def test_llama3_70b_layout_total():
    # 16 sequences x 32768 tokens x 8 KV heads x 80 layers at 164 B per token-head
    per_layer = A.cache_bytes(np.full(16, 32768), 8)
    assert per_layer == 16 * 8 * 2048 * 2624
    assert abs(80 * per_layer / 1e9 - 55.03) < 0.01


def test_fp16_decode_bytes():
    # fp16 control path: 512 B per token per KV head (the guide's payload with
    # 2-byte elements), one block-table entry per page including a partial one
    assert A.fp16_decode_bytes(np.array([37]), 12, 3) == 3 * 37 * 512 + 4 * 3 + 4 + 2 * (2 * 12 * 128)
    assert A.fp16_decode_bytes(np.array([16, 1]), 4, 1) == 17 * 512 + 4 * 2 + 8 + 2 * (2 * 2 * 4 * 128)
    # against the guide's payload formula for one layer
    ctx = np.array([100, 2000, 4096])
    kv = A.fp16_decode_bytes(ctx, 32, 8) - 4 * (-(-ctx // 16)).sum() - 4 * 3 - 2 * (2 * 3 * 32 * 128)
    assert kv == A.fp16_kv_bytes(1, 8, 128, int(ctx.sum()))


def test_fp8_decode_bytes():
    # FP8 path: 256 B per token per KV head (one byte per element), one
    # block-table entry per page, two fp32 scales per KV head
    assert A.fp8_decode_bytes(np.array([37]), 12, 3) == 3 * 37 * 256 + 4 * 3 + 4 + 8 * 3 + 2 * (2 * 12 * 128)
    ctx = np.array([100, 2000, 4096])
    kv = (A.fp8_decode_bytes(ctx, 32, 8) - 4 * (-(-ctx // 16)).sum() - 4 * 3 - 8 * 8
          - 2 * (2 * 3 * 32 * 128))
    assert kv == A.fp16_kv_bytes(1, 8, 128, int(ctx.sum()), bytes_per_elem=1)
    # half the fp16 payload
    assert 2 * kv == A.fp16_kv_bytes(1, 8, 128, int(ctx.sum()))


def test_mq_bytes():
    # one token per sequence: the decode bytes plus the B + 1 query-row offsets
    ctx = np.array([37, 100])
    assert A.mq_bytes(ctx, [1, 1], 12, 3) == A.decode_bytes(ctx, 12, 3) + 4 * 3
    # each extra token adds its Q row and O row (fp16, Hq x 128)
    assert A.mq_bytes(ctx, [4, 2], 12, 3) - A.mq_bytes(ctx, [1, 1], 12, 3) == 4 * 4 * 12 * 128


def test_kivi2_bytes():
    # 2-bit pages: 32 + 32 B of codes per token, 4 B of V metadata per token,
    # 512 B of K metadata per page = 100 B per token per KV head, 5.12x fp16
    assert A.K2_CHUNK_BYTES == 1600 and A.K2_CHUNK_BYTES / 16 == 32 + 32 + 4 + 32
    assert A.FP16_TOKEN_BYTES / (A.K2_CHUNK_BYTES / 16) == 5.12
    assert A.cache_bytes([37], 3, A.K2_CHUNK_BYTES) == 3 * (2 * 1600 + 5 * 512)
    b = A.decode_bytes(np.array([37]), 12, 3, A.K2_CHUNK_BYTES)
    assert b == A.cache_bytes([37], 3, A.K2_CHUNK_BYTES) + 4 * 2 + 4 + 2 * (2 * 12 * 128)


def test_append_step_bytes():
    """One token per sequence: read 512 B per KV head, then a 512-B tail write,
    or for a completed page 15 tail tokens read and a 2624-B chunk written;
    an empty sequence takes no token."""
    ctx = [1, 16, 17, 0]
    want = 2 * (3 * 512 + 2 * 512 + (15 * 512 + 2624))
    assert A.append_step_bytes(ctx, 2) == want == 25728


def test_unique_bytes_count_each_shared_chunk_once():
    """Brute force: enumerate the (physical page, KV head) chunks every sequence
    reads and count distinct ones."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        b, hkv, share = int(rng.integers(2, 9)), int(rng.integers(1, 5)), int(rng.integers(1, 6))
        ctx = rng.integers(1, 200, size=b)
        sharing = rng.random(b) < 0.5
        alias = np.where(sharing, np.minimum(share, ctx // 16), 0)
        chunks, next_id = set(), 1000
        logical_full = 0
        for i in range(b):
            for p in range(int(ctx[i]) // 16):
                pid = p if p < alias[i] else (next_id := next_id + 1)
                for h in range(hkv):
                    chunks.add((pid, h))
                logical_full += hkv
        logical = A.decode_bytes(ctx, 4 * hkv, hkv)
        unique = A.decode_bytes_unique(ctx, 4 * hkv, hkv, alias)
        assert logical - unique == (logical_full - len(chunks)) * A.CHUNK_BYTES
