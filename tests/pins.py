"""Pins: checks that tie the CPU oracle to facts fixed outside the oracle itself.

Each ``pin_*`` function takes an object ``o`` exposing the oracle's functions
(``quantize_groups``, ``dequantize``, ``flush_pages``, ``sequence_cache``,
``dequantized_sequence``, ``decode_attention``) and raises ``AssertionError``
when the oracle breaks the fact. ``test_oracle_pins.py`` runs them on the real
oracle; ``test_pins_catch_mistakes.py`` runs them on oracles with a planted
mistake (on the CPU) and requires that some pin fails, so that a plausible
error anywhere in the oracle cannot pass unnoticed.

The facts come from IEEE 754 binary16/binary32 arithmetic, closed forms of the
quantizer, brute force on tiny inputs and library routines (torch's
scaled_dot_product_attention), never from the oracle's own formulas.
"""

import math

import numpy as np

F16 = np.float16
F32 = np.float32


def _h(bits):
    """fp16 value from its bit pattern."""
    return np.array([bits], dtype=np.uint16).view(F16)[0]


# ---------------------------------------------------------------- quantizer

def pin_uniform_group(o):
    """All values equal: scale 0, zero = the value, codes 0, exact dequant."""
    for val in (0.0, 1.5, -3.25, 65504.0, 6e-8):
        x = np.full(16, val, dtype=F16)
        c, s, z = o.quantize_groups(x)
        assert np.all(c == 0), "uniform group must give code 0"
        assert s.view(np.uint16) == 0, "uniform group must give scale +0"
        assert z == F16(val), "zero point must be the value"
        xh = o.dequantize(c, s, z)
        assert np.all(xh == np.float32(F16(val))), "uniform group reconstructs exactly"


def pin_rne_ties():
    """Ties round to even (IEEE roundTiesToEven): with min 0 and max 15 the
    scale is exactly 1, so each code is the tie-to-even rounding of x."""
    x = np.array([0, 15, 2.5, 3.5, 0.5, 1.5, 4.5, 13.5, 14.5, 7.25, 7.75], dtype=F16)
    want = np.array([0, 15, 2, 4, 0, 2, 4, 14, 14, 7, 8], dtype=np.uint8)
    return x, want


def pin_rne(o):
    x, want = pin_rne_ties()
    c, s, z = o.quantize_groups(x)
    assert s == F16(1.0) and z == F16(0.0), "scale must be (15-0)/15 = 1, zero 0"
    assert np.array_equal(c, want), f"ties must round to even: got {c}, want {want}"


def pin_exact_grid(o, seed=0, trials=200):
    """Values lying exactly on a grid z + s*c (s a power of two times a short
    mantissa, codes covering 0 and 15) must be recovered exactly: codes, scale,
    zero, and the dequantized values."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        n = int(rng.choice([16, 128]))
        e = int(rng.integers(-8, 3))
        mant = int(rng.integers(1, 16))            # scale = mant * 2^e, 4-bit mantissa
        s = F32(mant) * F32(2.0) ** e
        z = F32(rng.integers(-64, 64)) * F32(2.0) ** (e)
        codes = rng.integers(0, 16, size=n).astype(np.uint8)
        codes[rng.integers(0, n)] = 0
        i15 = int(rng.integers(0, n))
        codes[i15] = 15
        if codes.min() != 0:
            codes[(i15 + 1) % n] = 0
        x = (z + s * codes.astype(F32)).astype(F16)
        assert np.array_equal(x.astype(F32), z + s * codes.astype(F32)), "grid must be exact"
        c, s16, z16 = o.quantize_groups(x)
        assert np.array_equal(c, codes), "grid codes must be recovered"
        assert F32(s16) == s and F32(z16) == z, "grid scale/zero must be recovered"
        assert np.array_equal(o.dequantize(c, s16, z16), x.astype(F32))


def pin_min_max_bound(o, seed=1, trials=300):
    """For random groups: code(min) = 0 and min reconstructs exactly;
    code(max) = 15; |x - x_hat| <= s/2 plus one fp32 rounding; codes in 0..15.
    Includes groups with outlier entries (x10..x20)."""
    rng = np.random.default_rng(seed)
    for i in range(trials):
        n = 16 if i % 2 else 128
        x = rng.standard_normal(n).astype(F32)
        if i % 3 == 0:
            x[rng.integers(0, n)] *= F32(rng.uniform(10, 20))
        x16 = x.astype(F16)
        c, s, z = o.quantize_groups(x16)
        assert c.dtype == np.uint8 and c.max() <= 15
        imin, imax = int(np.argmin(x16)), int(np.argmax(x16))
        assert z == x16[imin]
        assert c[imin] == 0
        xh = o.dequantize(c, s, z)
        assert xh[imin] == F32(x16[imin]), "the minimum must reconstruct exactly"
        if x16.max() > x16.min():
            assert c[imax] == 15, "the maximum must get code 15"
            s32 = F32(s)
            err = np.abs(x16.astype(np.float64) - xh.astype(np.float64))
            slack = 4 * np.spacing(np.abs(x16.astype(F32)).max())
            assert np.all(err <= s32 / 2 + slack), "error must be at most half a step"
            # the stored scale is the fp16 rounding of (max - min) / 15
            exact = (float(x16.max()) - float(x16.min())) / 15.0
            tol = float(np.spacing(F16(exact))) * 0.5 + 2 * float(np.spacing(F32(exact)))
            assert abs(float(s) - exact) <= tol, "scale must be (max - min) / 15 in fp16"


def pin_axes(o):
    """KEY is grouped per channel over the 16 tokens, VALUE per token over the
    channels: a K page whose channels are constant over tokens has all K scales
    0, a V page whose tokens are constant over channels has all V scales 0, and
    ramps along the group axis are recovered exactly."""
    d = 128
    rng = np.random.default_rng(7)
    kconst = np.tile(rng.integers(-8, 8, size=(1, d)).astype(F16), (16, 1))  # const over tokens
    vconst = np.tile(rng.integers(-8, 8, size=(16, 1)).astype(F16), (1, d))  # const over channels
    pg = o.flush_pages(kconst, vconst)
    assert np.all(pg["sk"] == 0) and np.all(pg["sv"] == 0)
    assert np.array_equal(pg["zk"], kconst[0]) and np.array_equal(pg["zv"], vconst[:, 0])
    # ramps: K[t, d] = zk[d] + sk[d] * t ; V[t, d] = zv[t] + sv[t] * perm_t(d) % 16
    sk = (2.0 ** rng.integers(-4, 2, size=d)).astype(F32)
    zk = rng.integers(-16, 16, size=d).astype(F32) / 4
    t = np.arange(16, dtype=F32)[:, None]
    k = (zk[None, :] + sk[None, :] * t).astype(F16)
    sv = (2.0 ** rng.integers(-4, 2, size=16)).astype(F32)
    zv = rng.integers(-16, 16, size=16).astype(F32) / 4
    cvw = np.stack([rng.permutation(np.arange(d) % 16) for _ in range(16)]).astype(np.uint8)
    v = (zv[:, None] + sv[:, None] * cvw.astype(F32)).astype(F16)
    pg = o.flush_pages(k, v)
    assert np.array_equal(pg["ck"], np.tile(np.arange(16, dtype=np.uint8)[:, None], (1, d)))
    assert np.array_equal(pg["sk"].astype(F32), sk) and np.array_equal(pg["zk"].astype(F32), zk)
    assert np.array_equal(pg["cv"], cvw)
    assert np.array_equal(pg["sv"].astype(F32), sv) and np.array_equal(pg["zv"].astype(F32), zv)


def pin_special_values(o):
    """Scale underflow, the clamp, and negative zero (IEEE binary16 facts)."""
    tiny = _h(0x0001)                                   # 2^-24, smallest subnormal
    # range 2^-24: (2^-24)/15 is below half the smallest subnormal -> scale 0
    x = np.array([0.0] * 8 + [tiny] * 8, dtype=F16)
    c, s, z = o.quantize_groups(x)
    assert s.view(np.uint16) == 0 and np.all(c == 0), "underflowing scale gives codes 0"
    # range 22*2^-24: 22/15 = 1.47 ulp rounds to 1 ulp, so (max-min)/s = 22 -> clamp 15
    x = np.array([0.0] * 15 + [F32(22) * F32(2.0 ** -24)], dtype=F16)
    c, s, z = o.quantize_groups(x)
    assert s.view(np.uint16) == 1, "scale must round to the smallest subnormal"
    assert c[-1] == 15 and np.all(c[:-1] == 0), "codes must clamp to 15"
    # negative zero as the minimum is stored as +0
    x = np.array([-0.0, 1.0, 2.0, 0.5] * 4, dtype=F16)
    c, s, z = o.quantize_groups(x)
    assert z.view(np.uint16) == 0, "zero point -0 must be stored as +0"
    x = np.array([-0.0] * 16, dtype=F16)
    c, s, z = o.quantize_groups(x)
    assert z.view(np.uint16) == 0 and s.view(np.uint16) == 0


# ---------------------------------------------------------------- cache state

def pin_cache_tail(o, seed=3):
    """Fewer than 16 tokens: no int4 page, the tail holds the exact fp16 tokens;
    a multiple of 16: no tail. Tokens on an exact grid (see pin_exact_grid)
    dequantize to themselves in order, so positions are checked exactly."""
    rng = np.random.default_rng(seed)
    hkv, d = 2, 128
    for ctx in (1, 7, 15):
        k = rng.standard_normal((ctx, hkv, d)).astype(F16)
        v = rng.standard_normal((ctx, hkv, d)).astype(F16)
        cache = o.sequence_cache(k, v)
        assert cache["full"] == 0
        kh, vh = o.dequantized_sequence(cache)
        assert np.array_equal(kh, k.astype(F32)) and np.array_equal(vh, v.astype(F32))
    for ctx in (16, 48, 53):
        codes_k = rng.integers(0, 16, size=(ctx, hkv, d)).astype(F32)
        codes_v = rng.integers(0, 16, size=(ctx, hkv, d)).astype(F32)
        # force 0 and 15 into every K channel group and V token group
        full = ctx // 16
        for p in range(full):
            codes_k[16 * p, :, :] = 0
            codes_k[16 * p + 1, :, :] = 15
        codes_v[:, :, 0] = 0
        codes_v[:, :, 1] = 15
        k = (codes_k * F32(0.25) - F32(2)).astype(F16)
        v = (codes_v * F32(0.125) + F32(1)).astype(F16)
        cache = o.sequence_cache(k, v)
        assert cache["full"] == full and cache["tail_k"].shape[0] == ctx - 16 * full
        kh, vh = o.dequantized_sequence(cache)
        assert np.array_equal(kh, k.astype(F32)), "grid K must reconstruct in token order"
        assert np.array_equal(vh, v.astype(F32)), "grid V must reconstruct in token order"


def pin_cache_prefix_stable(o, seed=4):
    """Appending tokens never changes an already full page (a page is
    quantized once, from its own 16 tokens)."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((70, 2, 128)).astype(F16)
    v = rng.standard_normal((70, 2, 128)).astype(F16)
    a = o.sequence_cache(k[:33], v[:33])
    b = o.sequence_cache(k, v)
    for key in ("ck", "sk", "zk", "cv", "sv", "zv"):
        assert np.array_equal(a["pages"][key], b["pages"][key][: a["full"]])


# ---------------------------------------------------------------- attention

def brute_force_attention(q, k, v, sm_scale):
    """Pure-Python decode attention with math.fsum; q [Hq][D], k/v [ctx][Hkv][D]."""
    hq, d = len(q), len(q[0])
    ctx, hkv = len(k), len(k[0])
    g = hq // hkv
    out = []
    for j in range(hq):
        h = j // g
        logits = [sm_scale * math.fsum(float(q[j][i]) * float(k[t][h][i]) for i in range(d))
                  for t in range(ctx)]
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        den = math.fsum(w)
        out.append([math.fsum(w[t] * float(v[t][h][i]) for t in range(ctx)) / den
                    for i in range(d)])
    return np.array(out)


def pin_attention_brute(o, seed=5):
    rng = np.random.default_rng(seed)
    for ctx, hq, hkv, d in ((1, 2, 1, 8), (5, 4, 2, 8), (23, 6, 2, 16), (40, 8, 8, 4)):
        q = rng.standard_normal((hq, d)).astype(F16)
        k = rng.standard_normal((ctx, hkv, d)).astype(F32) * 3
        v = rng.standard_normal((ctx, hkv, d)).astype(F32)
        sm = 1 / math.sqrt(d)
        got = o.decode_attention(q, k, v, sm)
        want = brute_force_attention(q.astype(np.float64).tolist(), k.tolist(), v.tolist(), sm)
        assert np.allclose(got, want, rtol=0, atol=1e-12), "attention vs brute force"


def pin_attention_sdpa(o, seed=6):
    """Library routine: torch scaled_dot_product_attention (CPU, float64, its
    default scale 1/sqrt(D)) with the K/V heads repeated over each query group."""
    import torch
    rng = np.random.default_rng(seed)
    hq, hkv, d, ctx = 8, 2, 128, 77
    q = rng.standard_normal((hq, d)).astype(F16)
    k = rng.standard_normal((ctx, hkv, d)).astype(F32)
    v = rng.standard_normal((ctx, hkv, d)).astype(F32)
    got = o.decode_attention(q, k, v)          # default scale: 1 / sqrt(head_dim)
    g = hq // hkv
    qt = torch.from_numpy(q.astype(np.float64))[:, None, :]                 # [Hq, 1, D]
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0, :].numpy()
    assert np.allclose(got, want, rtol=0, atol=1e-12), "attention vs torch SDPA"


def pin_attention_special(o, seed=8):
    rng = np.random.default_rng(seed)
    d = 128
    # one token: the output is that token's value
    q = rng.standard_normal((4, d)).astype(F16)
    k = rng.standard_normal((1, 1, d)).astype(F32)
    v = rng.standard_normal((1, 1, d)).astype(F32)
    assert np.allclose(o.decode_attention(q, k, v), np.repeat(v[:, 0, :], 4, 0), atol=1e-15)
    # zero query: uniform weights, output = mean of values
    k = rng.standard_normal((37, 1, d)).astype(F32)
    v = rng.standard_normal((37, 1, d)).astype(F32)
    out = o.decode_attention(np.zeros((2, d), F16), k, v)
    assert np.allclose(out, v[:, 0, :].astype(np.float64).mean(0), atol=1e-13)
    # one dominant key: output = its value
    qv = np.zeros((1, d), F16)
    qv[0, 0] = 8
    k = np.zeros((10, 1, d), F32)
    k[6, 0, 0] = 100.0     # logit gap 800/sqrt(128) = 70.7
    out = o.decode_attention(qv, k, v[:10])
    assert np.allclose(out[0], v[6, 0], atol=1e-13)
    # GQA grouping: query head j reads KV head j // G
    hkv, g = 4, 3
    v = np.zeros((5, hkv, d), F32)
    for h in range(hkv):
        v[:, h, :] = h + 1
    k = rng.standard_normal((5, hkv, d)).astype(F32)
    q = rng.standard_normal((hkv * g, d)).astype(F16)
    out = o.decode_attention(q, k, v)
    for j in range(hkv * g):
        assert np.allclose(out[j], j // g + 1, atol=1e-13), "query head j must read KV head j // G"
    # softmax scale: scale 2s on q equals scale s on 2q (doubling fp16 is exact)
    k = rng.standard_normal((20, 1, d)).astype(F32)
    v = rng.standard_normal((20, 1, d)).astype(F32)
    q = rng.standard_normal((1, d)).astype(F16)
    a = o.decode_attention(q, k, v, 0.2)
    b = o.decode_attention((q.astype(F32) * 2).astype(F16), k, v, 0.1)
    assert np.allclose(a, b, atol=1e-14)
    c = o.decode_attention(q, k, v, 0.1)
    assert not np.allclose(a, c, atol=1e-6), "the scale must enter the logits"


ALL_PINS = [
    pin_uniform_group,
    pin_rne,
    pin_exact_grid,
    pin_min_max_bound,
    pin_axes,
    pin_special_values,
    pin_cache_tail,
    pin_cache_prefix_stable,
    pin_attention_brute,
    pin_attention_sdpa,
    pin_attention_special,
]
