"""s4kv_paged_decode_append_noalloc (the decode step whose workspace is the
library's static per-device array, for callers that cannot allocate) against
s4kv_paged_decode_append with a caller-owned workspace, through the C ABI.

Two caches get the same prefill; each call of the allocation-free entry point
on one cache is matched by the workspace call on the other with the same new
token: outputs, pages and tails must agree bit for bit. Two calls in a row,
the second with a smaller input (fewer sequences, shorter contexts, another
group width), so the second call runs on the array the first one left
behind. A shape whose workspace exceeds the array is refused before any
launch."""

import ctypes

import numpy as np
import pytest
import torch

import workload as W
from int4_kivi_quantized_amd import Shape, s4kv
from tests.gpu_harness import LayerCase

pytestmark = pytest.mark.gpu


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _one_step(wl, steps, seed_step):
    ref = LayerCase(wl, extra_tokens=steps)
    noa = LayerCase(wl, extra_tokens=steps)
    for c in (ref, noa):
        c.prefill()
    ctx0 = ref.ctx.copy()
    max_ctx = int(ctx0.max()) + steps
    sm = 1.0 / np.sqrt(128.0)
    for s in range(steps):
        k, v = W.new_tokens(wl, 0, seed_step + s, "cuda", ref.mult)
        k, v = k.contiguous(), v.contiguous()
        ctx = torch.tensor((ctx0 + s + 1).astype(np.int32), device="cuda")
        want = ref.cache.decode_append(ref.q, k, v, ref.block_table, ctx, max_ctx)
        got = torch.empty_like(noa.q)
        s4kv.s4kv_paged_decode_append_noalloc(noa.shape, noa.q, k, v, noa.cache.pages,
                                              noa.cache.tail_k, noa.cache.tail_v, noa.block_table,
                                              ctx, max_ctx, sm, got)
        torch.cuda.synchronize()
        assert _same(got, want), f"{wl.name} step {s}: output differs"
        assert torch.equal(noa.cache.pages, ref.cache.pages), f"{wl.name} step {s}: pages differ"
        assert _same(noa.cache.tail_k, ref.cache.tail_k), f"{wl.name} step {s}: tail K differs"
        assert _same(noa.cache.tail_v, ref.cache.tail_v), f"{wl.name} step {s}: tail V differs"


def test_noalloc_matches_workspace_call_twice():
    big = W.Workload("noalloc-big", 1, 64, 32, 8, ("uniform", 2048, 8192),
                     ("frac", 0.02, 8.0, 20.0), append=True, seed=61)
    small = W.Workload("noalloc-small", 1, 5, 24, 8, ("uniform", 1, 300),
                       ("frac", 0.02, 8.0, 20.0), append=True, seed=62)
    for wl, steps in ((big, 3), (small, 17)):
        print(f"[case] noalloc workload={wl.name} B={wl.batch} G={wl.group} steps={steps}",
              flush=True)
        need = s4kv.s4kv_decode_workspace_bytes(
            Shape(wl.batch, wl.hq, wl.hkv, 1, 1024), 1024)
        assert need <= s4kv.NOALLOC_SCRATCH_BYTES
        _one_step(wl, steps, 100 * wl.seed)


def test_noalloc_refuses_shapes_beyond_the_array():
    # G = 16 and many (sequence, head) pairs: the partial slots exceed the array
    sh = Shape(num_seqs=4096, num_q_heads=256, num_kv_heads=16, num_pages=8, max_pages_per_seq=4)
    assert s4kv.s4kv_decode_workspace_bytes(sh, 64) > s4kv.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(16)   # never dereferenced: the call is refused on the host
    st = s4kv.load().s4kv_paged_decode_append_noalloc(ctypes.byref(sh.c()), *([fake] * 8), 64,
                                                       0.088, fake, None)
    assert st == s4kv.S4KV_ERR_SCRATCH_LIMIT
