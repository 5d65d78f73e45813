"""The append, decode and multi-query calls under HIP graph capture (torch.cuda.graph).

The C ABI allocates nothing and never synchronizes, so one decode step (append
one token per sequence, then decode) can be captured once and replayed: each
replay appends the next token (slot, context and token values are updated in
place between replays, with eager work and synchronizations in between) and
must give exactly what the same calls give eagerly, step after step.
"""

import numpy as np
import pytest
import torch

import workload as W
from tests.gpu_harness import LayerCase

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["int4", "kivi2", "fp8"])
def test_captured_step_replays_match_eager(kind):
    print(f"[case] captured_step kind={kind}", flush=True)
    base = W.WORKLOADS["llama3.2-3b-layer"]
    wl = W.Workload("graph-3b", 1, 16, base.hq, base.hkv, base.ctx, base.k_outliers, seed=base.seed)
    ctx0 = W.context_lengths(wl)
    steps = 6
    eager = LayerCase(wl, ctx_lens=ctx0, extra_tokens=steps, kind=kind)
    graph = LayerCase(wl, ctx_lens=ctx0, extra_tokens=steps, kind=kind)
    if kind == "fp8":
        graph.cache.k_scale.copy_(eager.cache.k_scale)
        graph.cache.v_scale.copy_(eager.cache.v_scale)
    eager.prefill()
    graph.prefill()
    max_ctx = int(ctx0.max()) + steps
    cu = torch.arange(wl.batch + 1, dtype=torch.int32, device="cuda")
    # inputs the graph reads, updated in place between replays
    slot = torch.tensor(ctx0.astype(np.int32), device="cuda")
    ctx = slot + 1
    k_in = torch.empty((wl.batch, wl.hkv, wl.head_dim), dtype=torch.float16, device="cuda")
    v_in = torch.empty_like(k_in)
    out = torch.empty_like(graph.q)
    graph.cache.workspace(max_ctx)
    # warm the library (device attributes are read once, outside any capture)
    eager.cache.decode(eager.q, eager.block_table, eager.ctx_gpu, max_ctx)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    k0, v0 = W.new_tokens(wl, 0, 100, "cuda", graph.mult)
    k_in.copy_(k0)
    v_in.copy_(v0)
    with torch.cuda.graph(g):
        graph.cache.append(k_in, v_in, cu, slot, 1, graph.block_table)
        graph.cache.decode(graph.q, graph.block_table, ctx, max_ctx, out=out)
    torch.cuda.synchronize()
    # capturing records the kernels without running them: replay s is step s

    for s in range(steps):
        k, v = W.new_tokens(wl, 0, s, "cuda", graph.mult)
        k_in.copy_(k)
        v_in.copy_(v)
        slot.copy_(torch.tensor((ctx0 + s).astype(np.int32), device="cuda"))
        ctx.copy_(slot + 1)
        g.replay()
        # eager twin of the same step, with its own buffers
        sl_e = torch.tensor((ctx0 + s).astype(np.int32), device="cuda")
        eager.cache.append(k.contiguous(), v.contiguous(), cu, sl_e, 1, eager.block_table)
        ref = eager.cache.decode(eager.q, eager.block_table, sl_e + 1, max_ctx)
        junk = torch.randn(1 << 16, device="cuda").sum()          # unrelated eager work
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out, ref), f"replay {s}: output differs from the eager step"
        assert torch.equal(graph.cache.pages, eager.cache.pages), f"replay {s}: pages differ"
        if kind != "fp8":
            assert torch.equal(graph.cache.tail_k, eager.cache.tail_k), f"replay {s}: tail K differs"
            assert torch.equal(graph.cache.tail_v, eager.cache.tail_v), f"replay {s}: tail V differs"


def test_captured_fused_step_replays_match_eager():
    """The fused call (s4kv_paged_decode_append) captured once and replayed:
    every replay appends the next token and attends, exactly as the same call
    made eagerly on a twin cache."""
    print("[case] captured_fused_step", flush=True)
    base = W.WORKLOADS["llama3.2-3b-layer"]
    wl = W.Workload("graph-fused-3b", 1, 16, base.hq, base.hkv, base.ctx, base.k_outliers, seed=base.seed)
    ctx0 = W.context_lengths(wl)
    steps = 18                                   # crosses a page completion for every sequence
    eager = LayerCase(wl, ctx_lens=ctx0, extra_tokens=steps)
    graph = LayerCase(wl, ctx_lens=ctx0, extra_tokens=steps)
    eager.prefill()
    graph.prefill()
    max_ctx = int(ctx0.max()) + steps
    ctx = torch.tensor((ctx0 + 1).astype(np.int32), device="cuda")
    k_in = torch.empty((wl.batch, wl.hkv, wl.head_dim), dtype=torch.float16, device="cuda")
    v_in = torch.empty_like(k_in)
    out = torch.empty_like(graph.q)
    graph.cache.workspace(max_ctx)
    eager.cache.decode(eager.q, eager.block_table, eager.ctx_gpu, max_ctx)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graph.cache.decode_append(graph.q, k_in, v_in, graph.block_table, ctx, max_ctx, out=out)
    torch.cuda.synchronize()

    for s in range(steps):
        k, v = W.new_tokens(wl, 0, s, "cuda", graph.mult)
        k_in.copy_(k)
        v_in.copy_(v)
        ctx.copy_(torch.tensor((ctx0 + s + 1).astype(np.int32), device="cuda"))
        g.replay()
        ctx_e = torch.tensor((ctx0 + s + 1).astype(np.int32), device="cuda")
        ref = eager.cache.decode_append(eager.q, k.contiguous(), v.contiguous(), eager.block_table,
                                        ctx_e, max_ctx)
        junk = torch.randn(1 << 16, device="cuda").sum()          # unrelated eager work
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(out, ref), f"replay {s}: output differs from the eager call"
        assert torch.equal(graph.cache.pages, eager.cache.pages), f"replay {s}: pages differ"
        assert torch.equal(graph.cache.tail_k, eager.cache.tail_k), f"replay {s}: tail K differs"
        assert torch.equal(graph.cache.tail_v, eager.cache.tail_v), f"replay {s}: tail V differs"


@pytest.mark.parametrize("max_q", [4, 12])
def test_captured_multiquery_replays_match_eager(max_q):
    """s4kv_paged_attention_mq captured once and replayed with new query values
    written in place between replays (eager work and synchronizations in
    between): every replay equals the same call made eagerly. With 3 query
    heads per KV head, 4 tokens fit one column tile (12 columns, the wide
    layout) and 12 tokens take three tiles per sequence."""
    print(f"[case] captured_multiquery max_q={max_q}", flush=True)
    base = W.WORKLOADS["llama3.2-3b-layer"]
    wl = W.Workload("graph-mq-3b", 1, 16, base.hq, base.hkv, base.ctx, base.k_outliers, seed=base.seed)
    case = LayerCase(wl)
    case.prefill()
    t_counts = np.minimum(np.array([max_q - (b % 3) for b in range(wl.batch)]), case.ctx)
    cu_q = torch.from_numpy(np.concatenate([[0], np.cumsum(t_counts)]).astype(np.int32)).cuda()
    total_q = int(t_counts.sum())
    max_ctx = int(case.ctx.max())
    q_in = torch.empty((total_q, wl.hq, wl.head_dim), dtype=torch.float16, device="cuda")
    out = torch.empty_like(q_in)
    q_in.copy_(W.normal_fp16((total_q, wl.hq, wl.head_dim), 900, "cuda"))
    case.cache.attend(q_in, cu_q, max_q, case.block_table, case.ctx_gpu, max_ctx, out=out)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        case.cache.attend(q_in, cu_q, max_q, case.block_table, case.ctx_gpu, max_ctx, out=out)
    torch.cuda.synchronize()
    for s in range(4):
        q = W.normal_fp16((total_q, wl.hq, wl.head_dim), 901 + s, "cuda")
        q_in.copy_(q)
        g.replay()
        junk = torch.randn(1 << 16, device="cuda").sum()          # unrelated eager work
        torch.cuda.synchronize()
        got = out.clone()
        ref = case.cache.attend(q.contiguous(), cu_q, max_q, case.block_table, case.ctx_gpu, max_ctx)
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(got, ref), f"replay {s}: output differs from the eager call"


def test_captured_fp16_decode_replays_match_eager():
    """The fp16 control decode captured once and replayed with new queries
    written in place: every replay equals the eager call."""
    print("[case] captured_fp16_decode", flush=True)
    base = W.WORKLOADS["llama3.2-3b-layer"]
    wl = W.Workload("graph-fp16-3b", 1, 16, base.hq, base.hkv, base.ctx, base.k_outliers, seed=base.seed)
    case = LayerCase(wl, kind="fp16")
    case.prefill()
    max_ctx = int(case.ctx.max())
    q_in = torch.empty_like(case.q)
    q_in.copy_(case.q)
    out = torch.empty_like(case.q)
    case.cache.decode(q_in, case.block_table, case.ctx_gpu, max_ctx, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        case.cache.decode(q_in, case.block_table, case.ctx_gpu, max_ctx, out=out)
    torch.cuda.synchronize()
    for s in range(4):
        q = W.normal_fp16(tuple(case.q.shape), 950 + s, "cuda")
        q_in.copy_(q)
        g.replay()
        junk = torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        got = out.clone()
        ref = case.cache.decode(q.contiguous(), case.block_table, case.ctx_gpu, max_ctx)
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(got, ref), f"replay {s}: output differs from the eager call"
