"""Reader (and, for checker self-tests, writer) of the library's page format,
written from the format description in include/s4kv.h -- independent of both
the HIP code and the oracle. Used to turn GPU page bytes into logical
(token, channel) codes and fp16 scale/zero bit patterns.
"""

import numpy as np

PAGE = 16
D = 128
CHUNK_BYTES = 2624
CHUNK_STRIDE = 2688
OFF_KC, OFF_VC, OFF_KS, OFF_KZ, OFF_VS, OFF_VZ = 0, 1024, 2048, 2304, 2560, 2592


def _k_nibble_map():
    """For each nibble index n = 2*byte + (high?1:0) in the K block: (token, channel)."""
    tok = np.empty(2 * 1024, dtype=np.int64)
    ch = np.empty(2 * 1024, dtype=np.int64)
    for l in range(64):
        t, g = l % 16, l // 16
        for m in range(4):
            for k in range(8):
                byte = 16 * l + 4 * m + k // 2
                n = 2 * byte + (k % 2)
                tok[n] = t
                ch[n] = 32 * m + 8 * g + 2 * (k % 4) + k // 4
    return tok, ch


def _v_nibble_map():
    tok = np.empty(2 * 1024, dtype=np.int64)
    ch = np.empty(2 * 1024, dtype=np.int64)
    for l in range(64):
        r, g = l % 16, l // 16
        for m in range(4):
            for k in range(8):
                byte = 16 * l + 4 * m + k // 2
                n = 2 * byte + (k % 2)
                tok[n] = 4 * g + 2 * (k % 2) + k // 4
                ch[n] = 16 * (2 * m + (k % 4) // 2) + r
    return tok, ch


K_TOK, K_CH = _k_nibble_map()
V_TOK, V_CH = _v_nibble_map()


def _nibbles(block):
    """uint8 [..., 1024] -> uint8 [..., 2048] (low nibble first)."""
    lo = block & 0x0F
    hi = block >> 4
    return np.stack([lo, hi], axis=-1).reshape(*block.shape[:-1], 2048)


def read_chunks(raw):
    """raw: uint8 [..., CHUNK_STRIDE] -> dict of logical arrays.

    ck, cv: uint8 [..., 16, 128] (token, channel); sk, zk: uint16 bit patterns
    [..., 128]; sv, zv: uint16 [..., 16]; pad: uint8 [..., 64].
    """
    raw = np.asarray(raw, dtype=np.uint8)
    lead = raw.shape[:-1]
    kn = _nibbles(raw[..., OFF_KC:OFF_KC + 1024])
    vn = _nibbles(raw[..., OFF_VC:OFF_VC + 1024])
    ck = np.zeros(lead + (PAGE, D), dtype=np.uint8)
    cv = np.zeros(lead + (PAGE, D), dtype=np.uint8)
    ck[..., K_TOK, K_CH] = kn
    cv[..., V_TOK, V_CH] = vn
    u16 = lambda a, b: np.ascontiguousarray(raw[..., a:b]).view(np.uint16)
    return {
        "ck": ck, "cv": cv,
        "sk": u16(OFF_KS, OFF_KS + 256), "zk": u16(OFF_KZ, OFF_KZ + 256),
        "sv": u16(OFF_VS, OFF_VS + 32), "zv": u16(OFF_VZ, OFF_VZ + 32),
        "pad": raw[..., CHUNK_BYTES:CHUNK_STRIDE],
    }


def write_chunk(ck, sk, zk, cv, sv, zv):
    """Logical page (one KV head) -> uint8 [CHUNK_STRIDE] (checker self-tests only)."""
    raw = np.zeros(CHUNK_STRIDE, dtype=np.uint8)
    kn = np.asarray(ck, dtype=np.uint8)[K_TOK, K_CH]
    vn = np.asarray(cv, dtype=np.uint8)[V_TOK, V_CH]
    raw[OFF_KC:OFF_KC + 1024] = kn[0::2] | (kn[1::2] << 4)
    raw[OFF_VC:OFF_VC + 1024] = vn[0::2] | (vn[1::2] << 4)
    raw[OFF_KS:OFF_KS + 256] = np.asarray(sk, dtype=np.float16).view(np.uint8)
    raw[OFF_KZ:OFF_KZ + 256] = np.asarray(zk, dtype=np.float16).view(np.uint8)
    raw[OFF_VS:OFF_VS + 32] = np.asarray(sv, dtype=np.float16).view(np.uint8)
    raw[OFF_VZ:OFF_VZ + 32] = np.asarray(zv, dtype=np.float16).view(np.uint8)
    return raw


# ---- FP8 (E4M3) pool: 4096 bytes per (page, KV head), operand order ----
FP8_CHUNK_BYTES = 4096


def fp8_byte_map():
    """For each byte of an FP8 chunk: (is_v, token, channel), from the format
    text: byte 1024 j + 16 L + i with L = 16 g + c holds K[c][32 (2j + i/8) +
    8g + i%8] for j < 2 and V[4g + i%4][16 (4(j-2) + i/4) + c] for j >= 2."""
    is_v = np.empty(FP8_CHUNK_BYTES, dtype=bool)
    tok = np.empty(FP8_CHUNK_BYTES, dtype=np.int64)
    ch = np.empty(FP8_CHUNK_BYTES, dtype=np.int64)
    for j in range(4):
        for L in range(64):
            g, c = L // 16, L % 16
            for i in range(16):
                n = 1024 * j + 16 * L + i
                if j < 2:
                    is_v[n], tok[n], ch[n] = False, c, 32 * (2 * j + i // 8) + 8 * g + i % 8
                else:
                    is_v[n], tok[n], ch[n] = True, 4 * g + i % 4, 16 * (4 * (j - 2) + i // 4) + c
    return is_v, tok, ch


def read_fp8_chunks(raw):
    """uint8 [..., 4096] -> (K codes, V codes), each uint8 [..., 16 tokens, 128 channels]."""
    raw = np.asarray(raw, dtype=np.uint8)
    is_v, tok, ch = fp8_byte_map()
    lead = raw.shape[:-1]
    k = np.zeros(lead + (PAGE, D), dtype=np.uint8)
    v = np.zeros(lead + (PAGE, D), dtype=np.uint8)
    k[..., tok[~is_v], ch[~is_v]] = raw[..., ~is_v]
    v[..., tok[is_v], ch[is_v]] = raw[..., is_v]
    return k, v


def write_fp8_chunk(kc, vc):
    """K and V codes uint8 [16, 128] -> one FP8 chunk, uint8 [4096]."""
    is_v, tok, ch = fp8_byte_map()
    out = np.empty(FP8_CHUNK_BYTES, dtype=np.uint8)
    out[~is_v] = np.asarray(kc, dtype=np.uint8)[tok[~is_v], ch[~is_v]]
    out[is_v] = np.asarray(vc, dtype=np.uint8)[tok[is_v], ch[is_v]]
    return out


# ---- 2-bit KIVI pool: 1600 data bytes + 64 padding per (page, KV head) ----
K2_CHUNK_BYTES, K2_CHUNK_STRIDE = 1600, 1664
K2_OFF_KC, K2_OFF_VC, K2_OFF_KS, K2_OFF_KZ, K2_OFF_VS, K2_OFF_VZ = 0, 512, 1024, 1280, 1536, 1568


def _k2_maps():
    """Code index n = 4 * byte + (bit offset within the byte) / 2 of a 2-bit
    code block -> (token, channel), from the header's text: lane L = 16 g + c
    owns bytes 8 L .. 8 L + 7 as words dd = 0, 1 (little endian); K word dd
    holds channel 32 m + 8 g + i (m = 2 dd + mm) of token c at bit 8 mm +
    2 (i >> 1) + 16 (i & 1); V word dd holds channel 16 (4 dd + s) + c of
    token 4 g + k at bit 4 s + 2 (k >> 1) + 16 (k & 1)."""
    ktok = np.empty(2048, dtype=np.int64)
    kch = np.empty(2048, dtype=np.int64)
    vtok = np.empty(2048, dtype=np.int64)
    vch = np.empty(2048, dtype=np.int64)
    for L in range(64):
        g, c = L // 16, L % 16
        for dd in range(2):
            word0 = 16 * (2 * L + dd)            # first code index of this 32-bit word
            for mm in range(2):
                for i in range(8):
                    n = word0 + (8 * mm + 2 * (i >> 1) + 16 * (i & 1)) // 2
                    ktok[n], kch[n] = c, 32 * (2 * dd + mm) + 8 * g + i
            for s in range(4):
                for k in range(4):
                    n = word0 + (4 * s + 2 * (k >> 1) + 16 * (k & 1)) // 2
                    vtok[n], vch[n] = 4 * g + k, 16 * (4 * dd + s) + c
    return ktok, kch, vtok, vch


K2_KTOK, K2_KCH, K2_VTOK, K2_VCH = _k2_maps()


def _codes2(block):
    """uint8 [..., 512] -> uint8 [..., 2048], lowest bits first within each byte."""
    return np.stack([(block >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(*block.shape[:-1], 2048)


def read_chunks2(raw):
    """raw: uint8 [..., 1664] (2-bit pool) -> the dict read_chunks returns."""
    raw = np.asarray(raw, dtype=np.uint8)
    lead = raw.shape[:-1]
    ck = np.zeros(lead + (PAGE, D), dtype=np.uint8)
    cv = np.zeros(lead + (PAGE, D), dtype=np.uint8)
    ck[..., K2_KTOK, K2_KCH] = _codes2(raw[..., K2_OFF_KC:K2_OFF_KC + 512])
    cv[..., K2_VTOK, K2_VCH] = _codes2(raw[..., K2_OFF_VC:K2_OFF_VC + 512])
    u16 = lambda a, b: np.ascontiguousarray(raw[..., a:b]).view(np.uint16)
    return {
        "ck": ck, "cv": cv,
        "sk": u16(K2_OFF_KS, K2_OFF_KS + 256), "zk": u16(K2_OFF_KZ, K2_OFF_KZ + 256),
        "sv": u16(K2_OFF_VS, K2_OFF_VS + 32), "zv": u16(K2_OFF_VZ, K2_OFF_VZ + 32),
        "pad": raw[..., K2_CHUNK_BYTES:K2_CHUNK_STRIDE],
    }


def write_chunk2(ck, sk, zk, cv, sv, zv):
    """Logical 2-bit page (one KV head) -> uint8 [1664] (checker self-tests only)."""
    raw = np.zeros(K2_CHUNK_STRIDE, dtype=np.uint8)
    for off, codes in ((K2_OFF_KC, np.asarray(ck, np.uint8)[K2_KTOK, K2_KCH]),
                       (K2_OFF_VC, np.asarray(cv, np.uint8)[K2_VTOK, K2_VCH])):
        q = codes.reshape(512, 4)
        raw[off:off + 512] = q[:, 0] | (q[:, 1] << 2) | (q[:, 2] << 4) | (q[:, 3] << 6)
    raw[K2_OFF_KS:K2_OFF_KS + 256] = np.asarray(sk, dtype=np.float16).view(np.uint8)
    raw[K2_OFF_KZ:K2_OFF_KZ + 256] = np.asarray(zk, dtype=np.float16).view(np.uint8)
    raw[K2_OFF_VS:K2_OFF_VS + 32] = np.asarray(sv, dtype=np.float16).view(np.uint8)
    raw[K2_OFF_VZ:K2_OFF_VZ + 32] = np.asarray(zv, dtype=np.float16).view(np.uint8)
    return raw
