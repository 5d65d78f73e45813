"""Pins of the FP8 (E4M3) oracle against the format definition and torch's own
float8_e4m3fn type (an independent implementation of the same OCP format)."""

import numpy as np
import pytest
import torch

from oracle import fp8


def _torch_values(codes):
    t = torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def test_all_256_codes_match_torch():
    codes = np.arange(256)
    ours = fp8.e4m3_value(codes)
    ref = _torch_values(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                                  # S.1111.111 only
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))   # -0 is 0x80


def test_landmark_values():
    v = fp8.e4m3_value([0x7E, 0x08, 0x07, 0x01, 0x38, 0x3F, 0x80, 0xFE])
    assert list(v[:6]) == [448.0, 2.0 ** -6, 7 * 2.0 ** -9, 2.0 ** -9, 1.0, 1.875]
    assert v[6] == 0.0 and np.signbit(v[6])
    assert v[7] == -448.0


def test_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    back = fp8.e4m3_encode(fp8.e4m3_value(codes).astype(np.float32))
    assert np.array_equal(back, codes.astype(np.uint8))


def test_encode_matches_torch_in_range():
    r = np.random.default_rng(3)
    y = np.concatenate([r.normal(0, 1, 20000), r.normal(0, 60, 20000),
                        r.uniform(-2.0 ** -6, 2.0 ** -6, 20000)]).astype(np.float32)
    y = y[np.abs(y) < 440]
    ours = fp8.e4m3_encode(y)
    ref = torch.tensor(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_ties_go_to_the_even_code():
    codes = np.arange(0x00, 0x7D)                          # every positive pair c, c + 1
    lo = fp8.e4m3_value(codes)
    hi = fp8.e4m3_value(codes + 1)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)   # midpoints exact in fp32
    got = fp8.e4m3_encode(mid).astype(np.int64)
    want = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(got, want)
    # just above / below a midpoint goes to the nearer code
    up = np.nextafter(mid, np.float32(np.inf))
    assert np.array_equal(fp8.e4m3_encode(up).astype(np.int64), codes + 1)


def test_saturation_and_sign():
    y = np.array([448, 448.5, 463.9, 464, 480, 1e6, 65504], dtype=np.float32)
    assert np.all(fp8.e4m3_encode(y) == 0x7E)
    assert np.all(fp8.e4m3_encode(-y) == 0xFE)
    z = fp8.e4m3_encode(np.array([0.0, -0.0, 2.0 ** -11, -2.0 ** -11], dtype=np.float32))
    assert list(z) == [0x00, 0x80, 0x00, 0x80]              # tiny values keep their sign


def test_subnormal_rounding():
    s = 2.0 ** -9
    y = np.array([0.5 * s, 1.5 * s, 2.5 * s, 7.5 * s, 7.49 * s], dtype=np.float32)
    assert list(fp8.e4m3_encode(y)) == [0, 2, 2, 8, 7]     # ties to even; 8 * 2^-9 is code 8


def test_quantize_with_scale():
    # 3.0 / 0.5 = 6.0 = 1.5 * 2^2: exponent field 9, mantissa 4
    assert fp8.quantize_fp8(np.array([3.0], dtype=np.float16), 0.5)[0] == (9 << 3) | 4
    # the division is one fp32 operation: 1/3 does not reach the encoder exactly
    y = np.float32(np.float16(1.0)) / np.float32(3.0)
    assert fp8.quantize_fp8(np.array([1.0], dtype=np.float16), 3.0)[0] == fp8.e4m3_encode(np.array([y]))[0]


def test_sequence_scales_are_per_head():
    r = np.random.default_rng(5)
    k = r.normal(0, 1, (40, 3, 128)).astype(np.float16)
    v = r.normal(0, 1, (40, 3, 128)).astype(np.float16)
    ks, vs = [0.5, 1.0, 0.03], [1.0, 0.02, 2.0]
    kc, vc = fp8.fp8_sequence(k, v, ks, vs)
    kh, vh = fp8.fp8_dequantized(kc, vc, ks, vs)
    for h in range(3):
        # relative error of an E4M3 rounding is at most 2^-4 of the value (normal range)
        big = np.abs(k[:, h].astype(np.float64)) / ks[h] >= 2.0 ** -6
        err = np.abs(kh[:, h] - k[:, h].astype(np.float64))[big]
        assert np.all(err <= 2.0 ** -4 * np.abs(k[:, h].astype(np.float64))[big] + 1e-12)
    assert np.array_equal(kc[:, 1], fp8.quantize_fp8(k[:, 1], 1.0))


class _NpProxy:
    def __init__(self, **overrides):
        self._o = overrides

    def __getattr__(self, name):
        return self._o[name] if name in self._o else getattr(np, name)


def test_pins_catch_planted_mistakes(monkeypatch):
    """Plausible slips in the encoder (rounding ties away from zero, no
    saturation, keeping only the magnitude) each break a pin above."""
    away = lambda x: np.sign(x) * np.floor(np.abs(x) + 0.5)
    monkeypatch.setattr(fp8, "np", _NpProxy(rint=away))
    with pytest.raises(AssertionError):
        test_ties_go_to_the_even_code()
    # no saturation at all: magnitudes past 448 run into the NaN code
    monkeypatch.setattr(fp8, "np", _NpProxy(minimum=lambda a, b: a))
    monkeypatch.setattr(fp8, "E4M3_MAX", float("inf"))
    with pytest.raises(AssertionError):
        test_saturation_and_sign()
    monkeypatch.setattr(fp8, "E4M3_MAX", 448.0)
    monkeypatch.setattr(fp8, "np", _NpProxy(signbit=lambda y: np.zeros(np.shape(y), dtype=bool)))
    with pytest.raises(AssertionError):
        test_saturation_and_sign()
