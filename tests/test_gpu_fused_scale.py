"""The fused decode step (s4kv_paged_decode_append) at the shapes it runs at
in the benchmark, through the C ABI.

A Llama-3.1-8B-shaped layer (B128, 32 query / 8 KV heads, contexts
U[2048, 8192]) holds about 330 000 units (full pages and tails) for the
persistent grid's 2048 waves, so every wave streams page pairs, and the page a
new token completes (S4 KV product page, "Funktionsweise" steps 1-2: the token
joins the fp16 tail, the page is quantized when its 16th token arrives) is
consumed either as page B of a pair or as a single page. Both happen at this
shape; a host replica of the unit split counts them and the test requires
both.

For layers 0 and 31 of that workload, and for a 70B-shaped head layout
(64 / 8, G = 8), two caches get the same prefill into junk-filled pools; then
17 steps append one token per sequence, one cache through the fused call, the
other through s4kv_quantize_append followed by s4kv_paged_decode. Pages, tails
and outputs must agree bit for bit at every step (17 steps pass at least one
page boundary in every sequence). After the last step every page and tail of
every sequence is compared bit-exactly with the oracle, and the output of
every sequence and query head is checked against the oracle's attention.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import workload as W
from tests import parity
from tests.gpu_harness import LayerCase
from tests.unit_split import completion_kinds

pytestmark = pytest.mark.gpu

STEPS = 17
TAIL_JUNK = 0x7E01   # a NaN bit pattern in the tail slots nobody wrote


def grid_waves():
    """Waves of the persistent decode grid: 8 per CU, at most 4096 (as the library sizes it)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return min(8 * cus, 4096)


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _run_fused_vs_separate(wl, layer, ctx0=None):
    sep = LayerCase(wl, layer=layer, ctx_lens=ctx0, extra_tokens=STEPS)
    fus = LayerCase(wl, layer=layer, ctx_lens=ctx0, extra_tokens=STEPS)
    ctx0 = sep.ctx.copy()
    for c in (sep, fus):
        c.cache.pages.fill_(0xAB)
        c.cache.tail_k.view(torch.int16).fill_(TAIL_JUNK)
        c.cache.tail_v.view(torch.int16).fill_(TAIL_JUNK)
        c.prefill()
    assert torch.equal(sep.cache.pages, fus.cache.pages)
    waves = grid_waves()
    max_ctx = int(ctx0.max()) + STEPS
    cu = torch.arange(wl.batch + 1, dtype=torch.int32, device="cuda")
    new = []
    kinds = np.zeros(2, dtype=np.int64)
    for s in range(STEPS):
        k, v = W.new_tokens(wl, layer, s, "cuda", sep.mult)
        k, v = k.contiguous(), v.contiguous()
        new.append((k, v))
        slot = torch.tensor((ctx0 + s).astype(np.int32), device="cuda")
        ctx = slot + 1
        kinds += completion_kinds(ctx0 + s + 1, wl.hkv, waves)
        sep.cache.append(k, v, cu, slot, 1, sep.block_table)
        want = sep.cache.decode(sep.q, sep.block_table, ctx, max_ctx)
        got = fus.cache.decode_append(fus.q, k, v, fus.block_table, ctx, max_ctx)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"step {s}: output differs from append + decode"
        assert torch.equal(fus.cache.pages, sep.cache.pages), f"step {s}: pages differ"
        assert _same_bits(fus.cache.tail_k, sep.cache.tail_k), f"step {s}: tail K differs"
        assert _same_bits(fus.cache.tail_v, sep.cache.tail_v), f"step {s}: tail V differs"
    print(f"  {STEPS} steps bit-identical; completed pages consumed as page B of a pair: "
          f"{kinds[0]}, as a single page: {kinds[1]} (grid {waves} waves)", flush=True)
    assert kinds[0] > 0 and kinds[1] > 0, "both completion routes must occur at this shape"
    return fus, ctx0, new, got


def _check_against_oracle(case, ctx0, new, out_gpu):
    """Every page and tail bit-exact, every output within the attention bar."""
    wl = case.wl
    case.ctx = ctx0 + STEPS
    kvs, chunks, tails = [], [], []
    for b in range(wl.batch):
        k0, v0 = W.sequence_kv(wl, case.layer, b, int(ctx0[b]), "cuda", case.mult)
        k = torch.cat([k0] + [x[0][b:b + 1] for x in new]).cpu().numpy()
        v = torch.cat([v0] + [x[1][b:b + 1] for x in new]).cpu().numpy()
        kvs.append((k, v))
        chunks.append(case.gpu_chunks(b))
        tails.append(case.gpu_tail(b))
    q = case.q.cpu().numpy()
    out = out_gpu.float().cpu().numpy()

    def one(b):
        c = oracle.sequence_cache(*kvs[b])
        bad = parity.page_mismatches(chunks[b], c["pages"])
        tk, tv = tails[b]
        tail_ok = (np.array_equal(tk.view(np.uint16), c["tail_k"].view(np.uint16))
                   and np.array_equal(tv.view(np.uint16), c["tail_v"].view(np.uint16)))
        kh, vh = oracle.dequantized_sequence(c)
        return bad, tail_ok, oracle.decode_attention(q[b], kh, vh)

    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(one, range(wl.batch)))
    for b, (bad, tail_ok, _) in enumerate(res):
        assert not bad, f"seq {b}: page fields differ from the oracle: {bad}"
        assert tail_ok, f"seq {b}: tail differs from the oracle"
    want = np.stack([r[2] for r in res])
    ok, max_abs, rel = parity.attention_ok(out, want)
    print(f"  oracle: {wl.batch} sequences x {wl.hq} heads, pages and tails bit-exact, "
          f"max_abs={max_abs:.2e} rel_l2={rel:.2e}", flush=True)
    assert ok, (max_abs, rel)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layer", [0, 31])
def test_fused_call_at_8b_shape(layer):
    wl = W.WORKLOADS["llama3.1-8b-decode"]
    print(f"[case] fused_scale workload={wl.name} layer={layer} steps={STEPS}", flush=True)
    fus, ctx0, new, out = _run_fused_vs_separate(wl, layer)
    _check_against_oracle(fus, ctx0, new, out)


@pytest.mark.timeout(600)
def test_fused_call_g8():
    """G = 8 (the 70B head layout, 64 / 8) at batch 16 with 8B-like contexts:
    about 41 000 units over the grid, pairs and both completion routes."""
    wl = W.Workload("llama3-70b-heads-append", 1, 16, 64, 8, ("uniform", 2048, 8192),
                    ("frac", 0.02, 8.0, 20.0), append=True, seed=41)
    print(f"[case] fused_scale workload={wl.name} layer=0 steps={STEPS}", flush=True)
    fus, ctx0, new, out = _run_fused_vs_separate(wl, 0)
    _check_against_oracle(fus, ctx0, new, out)
