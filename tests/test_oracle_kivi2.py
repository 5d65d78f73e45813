"""Pins of the oracle's 2-bit KIVI quantizer (codes 0..3, scale (max - min) / 3)
against closed forms and IEEE facts, and planted mistakes they must catch."""

import numpy as np
import pytest

import oracle.quant as oq
import oracle.cache as oc

F16, F32 = np.float16, np.float32


def pin_ties_and_extremes():
    # min 0, max 3: the scale is exactly 1, so codes are round-half-even of x
    x = np.array([0, 3, 0.5, 1.5, 2.5, 1.0, 2.0, 0.25], F16)
    c, s, z = oq.quantize_groups(x, bits=2)
    assert s == F16(1.0) and z == F16(0.0)
    assert list(c) == [0, 3, 0, 2, 2, 1, 2, 0]


def pin_exact_grid(seed=0):
    r = np.random.default_rng(seed)
    for _ in range(200):
        s = F16(2.0 ** int(r.integers(-8, 4)) * (1 + int(r.integers(0, 8)) / 8))
        z = F16(int(r.integers(-64, 64)) / 16)
        codes = r.integers(0, 4, 128)
        codes[:2] = [0, 3]                       # the group spans the full range
        x = (z.astype(F32) + codes.astype(F32) * s.astype(F32)).astype(F16)
        if not np.array_equal(x.astype(F32), z.astype(F32) + codes.astype(F32) * s.astype(F32)):
            continue                             # grid not exact in fp16
        c, s2, z2 = oq.quantize_groups(x, bits=2)
        assert s2 == s and z2 == z, (s, s2, z, z2)
        assert np.array_equal(c, codes)


def pin_bound(seed=1):
    r = np.random.default_rng(seed)
    x = (r.standard_normal((300, 16)) * r.uniform(0.01, 30, (300, 1))).astype(F16)
    c, s, z = oq.quantize_groups(x, axis=-1, bits=2)
    assert c.max() <= 3
    xh = oq.dequantize(c, s, z, axis=-1).astype(np.float64)
    sf = s.astype(np.float64)[:, None]
    # the stored fp16 scale rounds (max - min) / 3: within 2^-11 relative
    assert np.all(np.abs(xh - x.astype(np.float64)) <= 0.5 * sf * (1 + 2 ** -9) + 1e-6 * sf)
    # the minimum maps to code 0 and the maximum to code 3
    assert np.all(c[np.arange(300), x.argmin(1)] == 0)
    assert np.all(c[np.arange(300), x.argmax(1)] == 3)


def pin_scale_is_range_over_3():
    c, s, z = oq.quantize_groups(np.array([-1.5, 3.0, 0.0, 1.5], F16), bits=2)
    assert s == F16(1.5) and z == F16(-1.5) and list(c) == [0, 3, 1, 2]
    c, s, z = oq.quantize_groups(np.full(16, F16(0.7)), bits=2)
    assert s == 0 and np.all(c == 0) and z == F16(0.7)


def pin_subnormal_clamp():
    """fp16 subnormals are multiples of 2^-24: the range 7 * 2^-24 gives
    (7/3) * 2^-24, stored as 2 * 2^-24, so the maximum's quotient is 3.5, which
    rounds to 4 and must clamp to 3."""
    tiny = np.array([0, 7, 2, 5], np.uint16).view(F16)
    c, s, z = oq.quantize_groups(tiny, bits=2)
    assert s.view(np.uint16) == 2 and z == 0
    assert list(c) == [0, 3, 1, 2]          # 2/2 = 1, 5/2 = 2.5 -> 2 (ties to even)


def pin_cache_layout_2bit(seed=2):
    r = np.random.default_rng(seed)
    k = r.standard_normal((37, 2, 128)).astype(F16)
    v = r.standard_normal((37, 2, 128)).astype(F16)
    st = oc.sequence_cache(k, v, bits=2)
    assert st["full"] == 2 and st["tail_k"].shape[0] == 5
    assert st["pages"]["ck"].max() <= 3 and st["pages"]["cv"].max() <= 3
    kh, vh = oc.dequantized_sequence(st)
    assert np.array_equal(kh[32:], k[32:].astype(F32))          # the tail stays exact
    # K is grouped per channel over a page: channel 5 of page 1, head 0
    c, s, z = oq.quantize_groups(k[16:32, 0, 5], bits=2)
    assert np.array_equal(st["pages"]["ck"][1, 0, :, 5], c) and st["pages"]["sk"][1, 0, 5] == s


ALL = [pin_ties_and_extremes, pin_exact_grid, pin_bound, pin_scale_is_range_over_3,
       pin_subnormal_clamp, pin_cache_layout_2bit]


@pytest.mark.parametrize("pin", ALL, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


class _NpProxy:
    def __init__(self, **o):
        self._o = o

    def __getattr__(self, n):
        return self._o[n] if n in self._o else getattr(np, n)


@pytest.mark.parametrize("mistake", ["qmax_15", "range_over_4", "no_clamp", "round_half_up"])
def test_pins_catch_planted_mistakes(mistake, monkeypatch):
    if mistake == "qmax_15":
        monkeypatch.setattr(oq, "qmax_of", lambda bits=4: 15)
    elif mistake == "range_over_4":
        monkeypatch.setattr(oq, "qmax_of", lambda bits=4: 4 if bits == 2 else 15)
    elif mistake == "no_clamp":
        monkeypatch.setattr(oq, "np", _NpProxy(clip=lambda a, lo, hi: a))
    else:
        monkeypatch.setattr(oq, "np", _NpProxy(rint=lambda t: np.floor(t + 0.5)))
    failed = 0
    for pin in ALL:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed, f"planted mistake {mistake} passed every pin"
