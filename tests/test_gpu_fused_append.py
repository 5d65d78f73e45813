"""The decode call with its append fused in (s4kv_paged_decode_append) against
the two separate calls (s4kv_quantize_append of one token, then
s4kv_paged_decode), through the C ABI.

Two caches get the same prefill and the same tokens step after step, one
through each path. Pages, tails and outputs must agree bit for bit at every
step, across page completions at every offset, for several group widths; the
final pages and the attention output are also checked against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import workload as W
from tests import parity
from tests.gpu_harness import LayerCase

pytestmark = pytest.mark.gpu


def _wl(name, batch, g, hkv, seed):
    return W.Workload(name, 1, batch, g * hkv, hkv, ("fixed", 1), ("frac", 0.02, 8.0, 20.0), seed=seed)


@pytest.mark.parametrize("g", [1, 3, 4, 8, 16])
def test_fused_steps_match_separate_calls(g):
    print(f"[case] fused_append g={g}", flush=True)
    ctx0 = np.array([0, 1, 15, 16, 17, 31, 100, 255, 1000, 64], dtype=np.int64)
    steps = 20
    wl = _wl(f"fused-g{g}", len(ctx0), g, 2, seed=500 + g)
    sep = LayerCase(wl, ctx_lens=ctx0, extra_tokens=steps)
    fus = LayerCase(wl, ctx_lens=ctx0, extra_tokens=steps)
    for c in (sep, fus):
        c.cache.pages.fill_(0xAB)          # pages not yet written hold junk
        if ctx0.max() > 0:
            c.prefill()
    assert torch.equal(sep.cache.pages, fus.cache.pages)
    max_ctx = int(ctx0.max()) + steps
    cu = torch.arange(wl.batch + 1, dtype=torch.int32, device="cuda")
    new = []
    for s in range(steps):
        k, v = W.new_tokens(wl, 0, s, "cuda", sep.mult)
        k, v = k.contiguous(), v.contiguous()
        new.append((k, v))
        slot = torch.tensor((ctx0 + s).astype(np.int32), device="cuda")
        ctx = slot + 1
        sep.cache.append(k, v, cu, slot, 1, sep.block_table)
        want = sep.cache.decode(sep.q, sep.block_table, ctx, max_ctx)
        got = fus.cache.decode_append(fus.q, k, v, fus.block_table, ctx, max_ctx)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {s}: output differs from append + decode"
        assert torch.equal(fus.cache.pages, sep.cache.pages), f"step {s}: pages differ"
        assert torch.equal(fus.cache.tail_k, sep.cache.tail_k), f"step {s}: tail K differs"
        assert torch.equal(fus.cache.tail_v, sep.cache.tail_v), f"step {s}: tail V differs"
    # the oracle, after the last step
    fus.ctx = ctx0 + steps
    out = got.float().cpu().numpy()
    gots, wants = [], []
    for b in range(wl.batch):
        k0, v0 = W.sequence_kv(wl, 0, b, int(ctx0[b]), "cuda", sep.mult)
        k = torch.cat([k0] + [x[0][b:b + 1] for x in new]).cpu().numpy()
        v = torch.cat([v0] + [x[1][b:b + 1] for x in new]).cpu().numpy()
        c = oracle.sequence_cache(k, v)
        fus_full = int(fus.ctx[b]) // 16
        chunks = fus.cache.chunk_view()[torch.from_numpy(
            fus.plan.block_table[b, :fus_full].astype(np.int64)).cuda()].cpu().numpy()
        bad = parity.page_mismatches(chunks, c["pages"])
        assert not bad, f"seq {b}: {bad}"
        kh, vh = oracle.dequantized_sequence(c)
        gots.append(out[b])
        wants.append(oracle.decode_attention(fus.q[b].cpu().numpy(), kh, vh))
    ok, max_abs, rel = parity.attention_ok(np.stack(gots), np.stack(wants))
    print(f"  oracle max_abs={max_abs:.2e} rel_l2={rel:.2e}", flush=True)
    assert ok, (max_abs, rel)


def test_fused_call_skips_empty_sequences():
    """ctx_lens[b] = 0 in the fused call: no token is taken for b, its output is
    zero and its cache bytes are untouched; the other sequences are served."""
    print("[case] fused_append_empty", flush=True)
    ctx0 = np.array([5, 0, 15, 0], dtype=np.int64)
    wl = _wl("fused-empty", len(ctx0), 4, 2, seed=77)
    case = LayerCase(wl, ctx_lens=ctx0, extra_tokens=16)
    case.prefill()
    pages0 = case.cache.pages.clone()
    tk0, tv0 = case.cache.tail_k.clone(), case.cache.tail_v.clone()
    k, v = W.new_tokens(wl, 0, 0, "cuda", case.mult)
    ctx = torch.tensor([6, 0, 16, 0], dtype=torch.int32, device="cuda")
    out = case.cache.decode_append(case.q, k.contiguous(), v.contiguous(), case.block_table, ctx, 16)
    torch.cuda.synchronize()
    assert not out[1].any() and not out[3].any(), "empty sequences must give zero outputs"
    assert out[0].abs().sum() > 0 and out[2].abs().sum() > 0
    hk = wl.hkv
    tail_k = case.cache.tail_k.view(wl.batch, hk, 16, 128)
    tail_k0 = tk0.view(wl.batch, hk, 16, 128)
    for b in (1, 3):
        assert torch.equal(tail_k[b], tail_k0[b]), f"seq {b}: tail changed"
    # sequence 0 took its token into tail slot 5; sequence 2 completed its first page
    assert torch.equal(tail_k[0, :, 5], k[0]), "new token not in the tail"
    changed = (case.cache.chunk_view() != pages0.view_as(case.cache.chunk_view())).any(dim=-1)
    ids = set(int(x) for x in torch.nonzero(changed.any(dim=-1)).flatten().cpu())
    assert ids == {int(case.plan.block_table[2, 0])}, f"only seq 2's first page may change, got {ids}"
