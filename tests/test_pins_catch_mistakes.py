"""Plant plausible mistakes in the CPU oracle (on the CPU) and require that at
least one pin fails for each. This shows the pins constrain every step of the
oracle, not only the ones that happen to be easy to check."""

import types

import numpy as np
import pytest

import oracle
import oracle.attention as oatt
import oracle.cache as ocache
import oracle.quant as oquant
from tests import pins


class _NpProxy:
    """numpy with one function replaced, installed as ``np`` inside one oracle module."""

    def __init__(self, **overrides):
        self._o = overrides

    def __getattr__(self, name):
        if name in self._o:
            return self._o[name]
        return getattr(np, name)


def _ns():
    # look the functions up at call time so monkeypatched module globals apply
    return types.SimpleNamespace(
        quantize_groups=lambda *a, **k: oquant.quantize_groups(*a, **k),
        dequantize=lambda *a, **k: oquant.dequantize(*a, **k),
        flush_pages=lambda *a, **k: oquant.flush_pages(*a, **k),
        sequence_cache=lambda *a, **k: ocache.sequence_cache(*a, **k),
        dequantized_sequence=lambda *a, **k: ocache.dequantized_sequence(*a, **k),
        decode_attention=lambda *a, **k: oatt.decode_attention(*a, **k),
    )


def _some_pin_fails():
    o = _ns()
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            return True
    return False


def _swap(orig, x16, axis, bits=4):
    # K grouped per token instead of per channel
    if axis == -2:
        c, s, z = orig(x16, axis=-1, bits=bits)
        return c, s[..., :1].repeat(x16.shape[-1], -1)[..., : x16.shape[-1]], z[..., :1].repeat(x16.shape[-1], -1)
    return orig(x16, axis=axis, bits=bits)


def _mutants():
    orig_q = oquant.quantize_groups
    orig_dq = oquant.dequantize
    orig_cache = ocache.sequence_cache

    def keep_neg_zero(x16, axis=-1, bits=4):
        c, s, z = orig_q(x16, axis, bits)
        z = np.where(z == 0, np.float16(-0.0), z).astype(np.float16)
        return c, s, z

    def drop_zero_point(c, s, z, axis=-1):
        return orig_dq(c, s, np.zeros_like(z), axis)

    def tail_off_by_one(k16, v16):
        out = orig_cache(k16, v16)
        full = out["full"]
        if full and out["tail_k"].shape[0]:
            out["tail_k"] = k16[full * 16 - 1: -1].copy()
        return out

    def transposed_pages(k16, v16):
        out = orig_cache(k16, v16)
        for key in ("ck", "cv"):
            a = out["pages"][key]
            out["pages"][key] = a[..., ::-1, :].copy()     # tokens of a page reversed
        return out

    def codes_from_fp32_scale(x16, axis=-1, bits=4):
        # codes divided by the fp32 range / qmax instead of the stored fp16 scale
        qmax = oquant.qmax_of(bits)
        c, s16, z16 = orig_q(x16, axis, bits)
        xg = np.moveaxis(np.asarray(x16), axis, -1)
        s32 = (xg.max(-1).astype(np.float32) - xg.min(-1).astype(np.float32)) / np.float32(qmax)
        den = np.where(s32 == 0, np.float32(1), s32).astype(np.float32)
        t = (xg.astype(np.float32) - z16.astype(np.float32)[..., None]) / den[..., None]
        q = np.where((s16 == 0)[..., None], 0, np.clip(np.rint(t), 0, qmax))
        return np.moveaxis(q.astype(np.uint8), -1, axis), s16, z16

    def attn_wrong_group(q16, khat, vhat, sm_scale=None):
        # query head j reads KV head j % Hkv instead of j // G
        hq, hkv = q16.shape[0], khat.shape[1]
        g = hq // hkv
        order = np.array([(j % hkv) * g + (j // hkv) for j in range(hq)])
        out = oatt.__dict__["_orig"](q16[order], khat, vhat, sm_scale)
        return out[np.argsort(order)]

    return {
        "round_half_up": ("np", oquant, _NpProxy(rint=lambda t: np.floor(t + 0.5))),
        "no_clamp": ("np", oquant, _NpProxy(clip=lambda a, lo, hi: a)),
        "round_toward_zero": ("np", oquant, _NpProxy(rint=np.trunc)),
        "scale_over_16": ("qmax_of", oquant, lambda bits=4: 16 if bits == 4 else 4),
        "k_grouped_per_token": ("quantize_groups", oquant,
                                lambda x, axis=-1, bits=4: _swap(orig_q, x, axis, bits)),
        "keep_negative_zero": ("quantize_groups", oquant, keep_neg_zero),
        "codes_from_fp32_scale": ("quantize_groups", oquant, codes_from_fp32_scale),
        "dequant_drops_zero": ("dequantize", oquant, drop_zero_point),
        "tail_off_by_one": ("sequence_cache", ocache, tail_off_by_one),
        "page_tokens_reversed": ("sequence_cache", ocache, transposed_pages),
        "default_scale_not_inv_sqrt_d": ("math", oatt, types.SimpleNamespace(sqrt=lambda d: 1.0)),
        "exp_of_negated_logits": ("np", oatt, _NpProxy(exp=lambda x: np.exp(-x))),
        "gqa_modulo_mapping": ("decode_attention", oatt, attn_wrong_group),
    }


MUTANTS = _mutants()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, module, value = MUTANTS[name]
    if name == "gqa_modulo_mapping":
        monkeypatch.setitem(oatt.__dict__, "_orig", oatt.decode_attention)
    monkeypatch.setattr(module, attr, value)
    assert _some_pin_fails(), f"planted mistake '{name}' passed every pin"


def test_unmodified_oracle_passes_all_pins():
    assert not _some_pin_fails()
