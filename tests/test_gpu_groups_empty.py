"""Every query-group width the library instantiates (G = Hq / Hkv = 1..16),
each cache format, with empty sequences in the batch, through the C ABI.

Each decode kernel is a template over G; this sweep runs every instantiation
of the int4, 2-bit, fp16 and FP8 paths on a small ragged batch that includes
sequences with no cached tokens. Those get an all-zero output (the documented
result for ctx_lens[b] <= 0); every other output is held to the decode bar
(2e-3 max-abs, 1e-3 relative L2) against the oracle of its format. A batch in
which every sequence is empty gives zeros everywhere.
"""

import numpy as np
import pytest
import torch

import oracle
import workload as W
from oracle import fp8 as ofp8
from tests import parity
from tests.gpu_harness import LayerCase

pytestmark = pytest.mark.gpu

KINDS = ["int4", "kivi2", "fp16", "fp8"]
CTX = np.array([0, 37, 0, 16, 300, 1, 0, 33, 0], dtype=np.int64)


def _wl(name, batch, g, hkv, seed):
    return W.Workload(name, 1, batch, g * hkv, hkv, ("fixed", 1), ("frac", 0.02, 8.0, 20.0), seed=seed)


def _case(wl, kind, ctx, extra_tokens=0):
    case = LayerCase(wl, ctx_lens=ctx, kind=kind, extra_tokens=extra_tokens)
    # dense pools: undefined slots hold NaN, so a read of one would show
    if kind == "fp16":
        case.cache.pages.fill_(float("nan"))
    elif kind == "fp8":
        case.cache.pages.fill_(0x7F)
    return case


def _reference(case, b):
    """Oracle output [Hq, 128] of sequence b in the case's format."""
    q = case.q[b].cpu().numpy()
    if case.kind in ("int4", "kivi2"):
        return case.oracle_out(b)
    k, v = case.seq_kv(b)
    k, v = k.cpu().numpy(), v.cpu().numpy()
    if case.kind == "fp16":
        return oracle.decode_attention(q, k.astype(np.float32), v.astype(np.float32))
    kc, vc = ofp8.fp8_sequence(k, v, case.k_scale, case.v_scale)
    kh, vh = ofp8.fp8_dequantized(kc, vc, case.k_scale, case.v_scale)
    return oracle.decode_attention(q, kh, vh)


@pytest.mark.parametrize("g", list(range(1, 17)))
@pytest.mark.parametrize("kind", KINDS)
def test_group_width_with_empty_sequences(kind, g):
    print(f"[case] group_width kind={kind} g={g}", flush=True)
    wl = _wl(f"gw-{kind}-{g}", len(CTX), g, 2, seed=300 + g)
    case = _case(wl, kind, CTX)
    case.prefill()
    out = case.decode().float().cpu().numpy()
    assert np.isfinite(out).all(), "non-finite output"
    empty = CTX == 0
    assert not out[empty].any(), "an empty sequence has a non-zero output"
    got = np.concatenate([out[b] for b in np.flatnonzero(~empty)])
    want = np.concatenate([_reference(case, b) for b in np.flatnonzero(~empty)])
    ok, max_abs, rel = parity.attention_ok(got, want)
    print(f"  max_abs={max_abs:.2e} rel_l2={rel:.2e} outputs={len(got)}", flush=True)
    assert ok, f"attention out of tolerance: max_abs={max_abs:.3e} rel_l2={rel:.3e}"


@pytest.mark.parametrize("kind", KINDS)
def test_all_sequences_empty(kind):
    """No sequence has a cached token: nothing to stream, zeros everywhere.
    The pool still has a page per sequence (max_ctx only bounds the launch)."""
    print(f"[case] all_empty kind={kind}", flush=True)
    ctx = np.zeros(5, dtype=np.int64)
    wl = _wl(f"empty-{kind}", len(ctx), 4, 2, seed=7)
    case = _case(wl, kind, ctx, extra_tokens=16)
    case.q.normal_()
    out = case.decode(max_ctx=16)
    assert torch.isfinite(out).all()
    assert not out.float().abs().sum().item(), "all-empty batch gave a non-zero output"
