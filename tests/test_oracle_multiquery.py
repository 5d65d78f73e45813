"""Pins of the oracle's multi-query (causal) attention, against facts fixed
outside it: torch's scaled_dot_product_attention with a mask built by
torch.tril, the pinned one-token decode attention, brute force on tiny inputs,
and causality itself. Planted mistakes in the causal limit must fail a pin."""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from tests import pins


def _inputs(seed, t, ctx, hq=4, hkv=2, d=16):
    r = np.random.default_rng(seed)
    q = r.standard_normal((t, hq, d)).astype(np.float16)
    k = (r.standard_normal((ctx, hkv, d)) * 2).astype(np.float32)
    v = r.standard_normal((ctx, hkv, d)).astype(np.float32)
    return q, k, v


def pin_sdpa_bottom_right(mq):
    """torch SDPA over every query row at once, the boolean mask being
    torch.tril(ones(T, ctx), diagonal = ctx - T): row t keeps keys <= ctx - T + t."""
    for seed, (t, ctx) in enumerate([(1, 7), (3, 3), (4, 19), (6, 40)]):
        q, k, v = _inputs(seed, t, ctx, hq=6, hkv=3, d=32)
        got = mq(q, k, v)
        g = 2
        qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)           # [Hq, T, D]
        kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
        vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(g, 0)
        mask = torch.tril(torch.ones(t, ctx, dtype=torch.bool), diagonal=ctx - t)
        want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        assert np.allclose(got, want.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12), (t, ctx)


def pin_last_token_is_decode(mq):
    q, k, v = _inputs(11, 5, 33)
    got = mq(q, k, v)
    assert np.allclose(got[-1], A.decode_attention(q[-1], k, v), rtol=0, atol=1e-13)
    q1 = q[:1]
    assert np.allclose(mq(q1, k, v)[0], A.decode_attention(q1[0], k, v), rtol=0, atol=1e-13)


def pin_brute_force_prefixes(mq):
    q, k, v = _inputs(12, 3, 9, hq=2, hkv=1, d=8)
    got = mq(q, k, v)
    for t in range(3):
        n = 9 - 3 + t + 1
        want = pins.brute_force_attention(q[t].astype(np.float64).tolist(), k[:n].tolist(),
                                          v[:n].tolist(), 1 / math.sqrt(8))
        assert np.allclose(got[t], want, rtol=0, atol=1e-12), t


def pin_causality(mq):
    """Token t does not see positions after ctx - T + t, and does see that one."""
    q, k, v = _inputs(13, 4, 21)
    base = mq(q, k, v)
    for t in range(4):
        p = 21 - 4 + t
        k2, v2 = k.copy(), v.copy()
        k2[p + 1:] += 5.0
        v2[p + 1:] -= 3.0
        assert np.array_equal(mq(q, k2, v2)[t], base[t]), f"token {t} sees the future"
        v3 = v.copy()
        v3[p] += 1.0
        assert not np.allclose(mq(q, k, v3)[t], base[t], atol=1e-9), f"token {t} misses itself"


ALL = [pin_sdpa_bottom_right, pin_last_token_is_decode, pin_brute_force_prefixes, pin_causality]


@pytest.mark.parametrize("pin", ALL, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(A.multiquery_attention)


def _limited(shift=0, top_left=False, full=False):
    """A multi-query oracle with a planted mistake in the causal limit."""
    def mq(q16, khat, vhat, sm_scale=None):
        t_new, ctx = q16.shape[0], khat.shape[0]
        out = []
        for t in range(t_new):
            n = ctx if full else (t + 1 if top_left else ctx - t_new + t + 1 + shift)
            n = min(max(n, 1), ctx)
            out.append(A.decode_attention(q16[t], khat[:n], vhat[:n], sm_scale))
        return np.stack(out)
    return mq


@pytest.mark.parametrize("mistake", ["limit+1", "limit-1", "top_left", "no_mask"])
def test_pins_catch_planted_mistakes(mistake):
    mq = {"limit+1": _limited(shift=1), "limit-1": _limited(shift=-1),
          "top_left": _limited(top_left=True), "no_mask": _limited(full=True)}[mistake]
    failed = 0
    for pin in ALL:
        try:
            pin(mq)
        except AssertionError:
            failed += 1
    assert failed > 0, f"planted mistake {mistake} passed every pin"
