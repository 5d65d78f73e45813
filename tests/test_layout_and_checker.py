"""The page-format reader covers every nibble exactly once, and the parity
checker fails on planted faults (the injected-fault self-test idea of the FP8
KV-cache guide, adechristanto.de, section on paired quality checks: a checker
is trusted only after it rejects known-bad results). CPU only."""

import math

import numpy as np

import oracle
from tests import layout, parity


def test_nibble_maps_are_bijections():
    for tok, ch in ((layout.K_TOK, layout.K_CH), (layout.V_TOK, layout.V_CH)):
        pairs = tok * 128 + ch
        assert np.array_equal(np.sort(pairs), np.arange(16 * 128))


def _oracle_page(seed=0):
    r = np.random.default_rng(seed)
    k = (r.standard_normal((16, 128)) * np.where(r.random(128) < 0.03, 12, 1)).astype(np.float16)
    v = r.standard_normal((16, 128)).astype(np.float16)
    return oracle.flush_pages(k, v)


def test_write_read_roundtrip():
    pg = _oracle_page()
    raw = layout.write_chunk(pg["ck"], pg["sk"], pg["zk"], pg["cv"], pg["sv"], pg["zv"])
    assert parity.page_mismatches(raw[None, None], {k: v[None, None] for k, v in pg.items()}) == []


def test_checker_catches_flipped_nibble():
    pg = _oracle_page(1)
    raw = layout.write_chunk(pg["ck"], pg["sk"], pg["zk"], pg["cv"], pg["sv"], pg["zv"])
    want = {k: v[None, None] for k, v in pg.items()}
    for off in (0, 517, 1023, 1024, 2047):
        bad = raw.copy()
        bad[off] ^= 0x10
        assert parity.page_mismatches(bad[None, None], want), f"flip at {off} not caught"


def test_checker_catches_one_ulp_scale():
    pg = _oracle_page(2)
    raw = layout.write_chunk(pg["ck"], pg["sk"], pg["zk"], pg["cv"], pg["sv"], pg["zv"])
    want = {k: v[None, None] for k, v in pg.items()}
    for off in (layout.OFF_KS + 2 * 5, layout.OFF_KZ, layout.OFF_VS + 2 * 15, layout.OFF_VZ + 2):
        bad = raw.copy()
        u = bad[off:off + 2].view(np.uint16)
        u[0] += 1
        assert parity.page_mismatches(bad[None, None], want), f"1-ulp change at {off} not caught"


def test_checker_catches_attention_faults():
    r = np.random.default_rng(3)
    q = r.standard_normal((8, 128)).astype(np.float16)
    k = r.standard_normal((300, 2, 128)).astype(np.float16)
    v = r.standard_normal((300, 2, 128)).astype(np.float16)
    c = oracle.sequence_cache(k, v)
    kh, vh = oracle.dequantized_sequence(c)
    ref = oracle.decode_attention(q, kh, vh)
    ok, _, _ = parity.attention_ok(ref.astype(np.float16).astype(np.float64), ref)
    assert ok, "fp16 rounding of the output alone must pass"
    bumped = ref.copy()
    bumped[3, 77] += 3e-3
    assert not parity.attention_ok(bumped, ref)[0], "a 3e-3 error must fail"
    # a block-table entry pointing at another sequence's page (attention is
    # order-free, so a swap inside one sequence is invisible; a foreign page is not)
    other = oracle.dequantized_sequence(oracle.sequence_cache(
        r.standard_normal((48, 2, 128)).astype(np.float16), r.standard_normal((48, 2, 128)).astype(np.float16)))
    kh2, vh2 = kh.copy(), vh.copy()
    kh2[32:48], vh2[32:48] = other[0][32:48], other[1][32:48]
    foreign = oracle.decode_attention(q, kh2, vh2)
    assert not parity.attention_ok(foreign, ref)[0], "a foreign page must fail"
    # a dropped tail token
    short = oracle.decode_attention(q, kh[:-1], vh[:-1])
    assert not parity.attention_ok(short, ref)[0], "a missing token must fail"
    # a wrong softmax scale
    wrong = oracle.decode_attention(q, kh, vh, sm_scale=1.0 / math.sqrt(64))
    assert not parity.attention_ok(wrong, ref)[0]


def test_fp8_byte_map_is_a_bijection():
    is_v, tok, ch = layout.fp8_byte_map()
    for v in (False, True):
        cells = set(zip(tok[is_v == v].tolist(), ch[is_v == v].tolist()))
        assert len(cells) == 16 * 128 and (is_v == v).sum() == 16 * 128
    # a lane's 16 bytes of a K block are channels 32m + 8g .. +7 of one token, m = 2j, 2j + 1
    assert list(ch[16 * 17:16 * 17 + 8]) == list(range(8, 16)) and set(tok[16 * 17:16 * 18]) == {1}
    # a lane's V bytes 4t' .. 4t'+3 are tokens 4g .. 4g+3 of one channel
    n = 2048 + 16 * 33 + 4
    assert list(tok[n:n + 4]) == [8, 9, 10, 11] and set(ch[n:n + 4]) == {16 + 1}


def test_fp8_write_read_roundtrip():
    r = np.random.default_rng(0)
    kc = r.integers(0, 256, (16, 128), dtype=np.uint8)
    vc = r.integers(0, 256, (16, 128), dtype=np.uint8)
    raw = layout.write_fp8_chunk(kc, vc)
    k2, v2 = layout.read_fp8_chunks(raw[None])
    assert np.array_equal(k2[0], kc) and np.array_equal(v2[0], vc)


def test_k2_code_maps_are_bijections():
    for tok, ch in ((layout.K2_KTOK, layout.K2_KCH), (layout.K2_VTOK, layout.K2_VCH)):
        assert len(set(zip(tok.tolist(), ch.tolist()))) == 16 * 128
    # lane 17 (g = 1, c = 1), word 0: K bits 0-1 are channel 8 of token 1, bits
    # 16-17 channel 9, bits 8-9 channel 32 + 8
    n0 = 16 * (2 * 17)
    assert (layout.K2_KTOK[n0], layout.K2_KCH[n0]) == (1, 8)
    assert (layout.K2_KTOK[n0 + 8], layout.K2_KCH[n0 + 8]) == (1, 9)
    assert (layout.K2_KTOK[n0 + 4], layout.K2_KCH[n0 + 4]) == (1, 40)
    # V word 1 of lane 33 (g = 2, c = 1): bits 4-5 are channel 16 * 5 + 1 of token 8
    n1 = 16 * (2 * 33 + 1)
    assert (layout.K2_VTOK[n1 + 2], layout.K2_VCH[n1 + 2]) == (8, 81)


def test_k2_write_read_roundtrip_and_checker():
    r = np.random.default_rng(4)
    k = r.standard_normal((16, 128)).astype(np.float16)
    v = r.standard_normal((16, 128)).astype(np.float16)
    pg = oracle.flush_pages(k, v, bits=2)
    raw = layout.write_chunk2(pg["ck"], pg["sk"], pg["zk"], pg["cv"], pg["sv"], pg["zv"])
    got = layout.read_chunks2(raw[None])
    assert np.array_equal(got["ck"][0], pg["ck"]) and np.array_equal(got["cv"][0], pg["cv"])
    want = {kk: vv[None, None] for kk, vv in pg.items()}
    assert parity.page_mismatches(raw[None, None], want, bits=2) == []
    bad = raw.copy()
    bad[700] ^= 0x04                                   # one V code changes
    assert parity.page_mismatches(bad[None, None], want, bits=2)
