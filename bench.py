"""Benchmark of the int4 KIVI paged KV cache on one MI355X.

A step is one decode step of the whole model-shaped stack: for every layer,
one new token per sequence is appended (fp16 tail, page quantized when its
16th token arrives) and attention runs over the int4 pages and the tail. By
default each layer's step is one s4kv_paged_decode_append call (append and
decode in one launch of the decode stream, then the split merge);
--separate-append times s4kv_quantize_append followed by s4kv_paged_decode
instead. Inputs (caches, queries, new tokens, context lengths) are resident
in HBM before the timed region. Each timed step (all layers' calls) is
captured in a HIP graph beforehand and replayed; the same steps launched
eagerly from Python are timed beside it (--eager times those alone).

Headline workload: Llama-3.1-8B-shaped decode, 32 layers, 32 query / 8 KV
heads, head_dim 128, batch 128, contexts U[2048, 8192], page 16.
Secondary (same JSON line): Llama-3-70B-shaped decode, 80 layers, 64/8 heads,
batch 16, 32768-token contexts, with the bulk prefill quantize of those
contexts timed separately; the same decode call over this library's 2-bit
KIVI, fp16 (control) and FP8 E4M3 caches against the int4 call, on one layer of the
headline workload; and multi-query attention (4 new tokens per sequence, the
speculative-verify step) against the decode call on that layer.

Two ceilings frame the decode call's rate: a copy (torch, read + write) and
the library's read probe (s4kv_probe_read: random 4 KB chunks through the
decode kernels' own load path, with and without the non-temporal policy).

Prints one JSON line. `value` is KV GB/s: the algorithmic bytes of all decode
launches of a step (pages, tails, block-table entries, Q, O) divided by the
step time. With the fused call a launch's bytes include its one-token append
(about 1.7 MB per 8B-shaped layer step: the new tokens, tail slots, and the
pages they complete); with --separate-append the append kernel's bytes are
not counted (its time is).
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workload as W  # noqa: E402
from workload import accounting as A  # noqa: E402

METRIC = "int4 paged-decode KV GB/s + % of HBM peak; decode tokens/s at 8B/70B shapes"
HBM_PEAK_GBS = 8000.0


def _sources_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "int4_kivi_quantized_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


class Model:
    """All layers of one workload: per-layer caches over one shared block table."""

    def __init__(self, wl, extra_steps, time_prefill=False):
        import torch
        from int4_kivi_quantized_amd import Shape
        from int4_kivi_quantized_amd.cache import LayerCache

        self.wl = wl
        self.ctx0 = W.context_lengths(wl)
        self.plan = W.plan_pages(wl, self.ctx0, extra_steps)
        self.shape = Shape(wl.batch, wl.hq, wl.hkv, self.plan.num_pages, self.plan.max_pages)
        self.bt = torch.from_numpy(self.plan.block_table).cuda()
        self.layers = []
        self.q = []
        self.mults = []
        self.prefill_ms = 0.0
        self.prefill_bytes = 0
        counts = self.ctx0.astype(np.int64)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device="cuda")
        sl = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
        for layer in range(wl.layers):
            cache = LayerCache(self.shape)
            mult = W.k_channel_multipliers(wl, layer)
            ks, vs = [], []
            for b in range(wl.batch):
                k, v = W.sequence_kv(wl, layer, b, int(self.ctx0[b]), "cuda", mult)
                ks.append(k)
                vs.append(v)
            k_all = torch.cat(ks).contiguous()
            v_all = torch.cat(vs).contiguous()
            del ks, vs
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            cache.append(k_all, v_all, cu, sl, int(counts.max()), self.bt)
            e1.record()
            torch.cuda.synchronize()
            if time_prefill:
                self.prefill_ms += e0.elapsed_time(e1)
                full = (counts // 16) * 16
                self.prefill_bytes += A.quantize_bytes(int(full.sum()), int((counts - full).sum()), wl.hkv)
            del k_all, v_all
            self.layers.append(cache)
            self.q.append(W.queries(wl, layer, "cuda"))
            self.mults.append(mult)
            if (layer + 1) % 16 == 0 or layer + 1 == wl.layers:
                print(f"[bench] {wl.name}: {layer + 1}/{wl.layers} layers prefilled",
                      file=sys.stderr, flush=True)
        torch.cuda.synchronize()


def run_decode_bench(wl, steps, warmup, append, fused=True, graph=True):
    import torch

    # warm-up steps; `steps` steps timed as eager launches; with `graph`, as
    # many steps again, each captured in a HIP graph beforehand and timed as
    # graph replays (the headline); then as many steps with HIP events around
    # every call for the per-call figures. Every step appends at its own
    # position, so each timed step does a step's full work.
    total = warmup + (3 if graph else 2) * steps
    model = Model(wl, total if append else 0, time_prefill=not append)
    B = wl.batch
    max_ctx = int(model.ctx0.max()) + (total if append else 0)
    cu1 = torch.arange(B + 1, dtype=torch.int32, device="cuda")
    slots, ctxs, new = [], [], []
    for s in range(total):
        add = s if append else 0
        slots.append(torch.tensor((model.ctx0 + add).astype(np.int32), device="cuda"))
        ctxs.append(torch.tensor((model.ctx0 + add + (1 if append else 0)).astype(np.int32), device="cuda"))
    if append:
        for layer in range(wl.layers):
            # one pre-drawn new token per sequence and layer, appended every step
            k, v = W.new_tokens(wl, layer, 0, "cuda", model.mults[layer])
            new.append((k.contiguous(), v.contiguous()))
    outs = [torch.empty_like(q) for q in model.q]
    for c in model.layers:
        c.workspace(max_ctx)
    torch.cuda.synchronize()

    n_ev = steps * wl.layers
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]

    def step(s, timed_idx=None):
        for layer, cache in enumerate(model.layers):
            if append and not fused:
                cache.append(new[layer][0], new[layer][1], cu1, slots[s], 1, model.bt)
            if timed_idx is not None:
                ev_a[timed_idx * wl.layers + layer].record()
            if append and fused:
                cache.decode_append(model.q[layer], new[layer][0], new[layer][1], model.bt, ctxs[s],
                                    max_ctx, out=outs[layer])
            else:
                cache.decode(model.q[layer], model.bt, ctxs[s], max_ctx, out=outs[layer])
            if timed_idx is not None:
                ev_b[timed_idx * wl.layers + layer].record()

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    graphs = []
    if graph:
        # one graph per step (the steps' context lengths differ); capturing
        # launches nothing
        for i in range(steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(warmup + steps + i)
            graphs.append(g)
        torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(steps):
        step(warmup + i)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    eager_ms = t0.elapsed_time(t1) / steps
    step_ms = eager_ms
    timed0 = warmup
    if graph:
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        g0.record()
        for g in graphs:
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        step_ms = g0.elapsed_time(g1) / steps
        timed0 = warmup + steps
    del graphs
    # per-call durations: the next `steps` steps, each call between two events
    ev0 = total - steps
    for i in range(steps):
        step(ev0 + i, i)
    torch.cuda.synchronize()
    dec_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]))

    # algorithmic bytes of the decode launches, per layer, averaged over timed steps
    # (with the fused call, the launch's bytes also count its one-token append)
    def layer_bytes(s):
        ctx_s = model.ctx0 + (s + 1 if append else 0)
        nb = A.decode_bytes(ctx_s, wl.hq, wl.hkv)
        if append and fused:
            nb += A.append_step_bytes(ctx_s, wl.hkv)
        return nb
    per_layer = [layer_bytes(timed0 + i) for i in range(steps)]            # timed steps
    per_call = [layer_bytes(ev0 + i) for i in range(steps)]                # per-call steps
    step_bytes = float(np.mean(per_layer)) * wl.layers
    dec_bytes = float(np.mean(per_call))
    res = {
        "step_ms": step_ms,
        "eager_step_ms": eager_ms,
        "graph": graph,
        "step_bytes": step_bytes,
        "wall_s": wall,
        "kv_gbs": step_bytes / (step_ms * 1e-3) / 1e9,
        "tokens_per_s": B / (step_ms * 1e-3),
        "decode_launch_ms": dec_ms,
        "decode_launch_bytes": dec_bytes,
        "decode_launch_gbs": dec_bytes / (dec_ms * 1e-3) / 1e9,
        "model": model,
    }
    if not append:
        res["prefill_gbs"] = model.prefill_bytes / (model.prefill_ms * 1e-3) / 1e9 if model.prefill_ms else None
        res["prefill_ms_per_layer"] = model.prefill_ms / wl.layers
    return res


def prefill_layer(cache, wl, layer, ctx, plan, bt):
    """Bulk prefill of one layer's int4 cache through s4kv_quantize_append: a
    shared prefix (if the workload has one) once into its physical pages, then
    every sequence's own tokens (after its aliased prefix pages)."""
    import torch
    from int4_kivi_quantized_amd import Shape
    from int4_kivi_quantized_amd.cache import LayerCache
    mult = W.k_channel_multipliers(wl, layer)
    alias = np.zeros(wl.batch, dtype=np.int64)
    if len(plan.sharing):
        share_pages = wl.shared_prefix // wl.page
        pk, pv = W.prefix_kv(wl, layer, "cuda", mult)
        pshape = Shape(1, wl.hq, wl.hkv, plan.num_pages, share_pages)
        scratch = LayerCache(Shape(1, wl.hq, wl.hkv, 1, share_pages))
        pbt = torch.from_numpy(plan.prefix_pages[None, :].copy()).cuda()
        from int4_kivi_quantized_amd import s4kv
        s4kv.s4kv_quantize_append(pshape, pk.contiguous(), pv.contiguous(),
                                  torch.tensor([0, wl.shared_prefix], dtype=torch.int32, device="cuda"),
                                  torch.zeros(1, dtype=torch.int32, device="cuda"), wl.shared_prefix,
                                  pbt, cache.pages, scratch.tail_k, scratch.tail_v)
        for b in plan.sharing:
            alias[b] = min(share_pages, int(ctx[b]) // wl.page)
    ks, vs, starts, counts = [], [], [], []
    for b in range(wl.batch):
        k, v = W.sequence_kv(wl, layer, b, int(ctx[b]), "cuda", mult)
        st = int(alias[b]) * wl.page
        ks.append(k[st:])
        vs.append(v[st:])
        starts.append(st)
        counts.append(int(ctx[b]) - st)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device="cuda")
    sl = torch.tensor(np.asarray(starts, dtype=np.int32), device="cuda")
    cache.append(torch.cat(ks).contiguous(), torch.cat(vs).contiguous(), cu, sl, max(counts), bt)
    torch.cuda.synchronize()
    return alias


def small_configs(calls=20, warmup=3):
    """The configurations checked for correctness, also reported in KV GB/s:
    the tiny case (one 256-token sequence: latency-bound); the 3B-shaped
    layer over 8 replicas called in rotation (its 97 MB cache fits in the
    256 MB last-level cache, so back-to-back calls on one copy would read it
    from there); the shared-prefix layer over 4 replicas in rotation, with
    logical bytes (every sequence's pages, shared ones once per reader) and
    unique bytes (each shared page once). Decode calls (s4kv_paged_decode),
    each between two HIP events on its stream; medians."""
    import torch
    from int4_kivi_quantized_amd import Shape
    from int4_kivi_quantized_amd.cache import LayerCache

    out = {}
    for name, reps in (("tiny", 1), ("llama3.2-3b-layer", 8), ("qwen2.5-7b-shared-prefix", 4)):
        wl = W.WORKLOADS[name]
        ctx = W.context_lengths(wl)
        plan = W.plan_pages(wl, ctx)
        shape = Shape(wl.batch, wl.hq, wl.hkv, plan.num_pages, plan.max_pages)
        bt = torch.from_numpy(plan.block_table).cuda()
        ctx_g = torch.from_numpy(ctx.astype(np.int32)).cuda()
        q = W.queries(wl, 0, "cuda")
        caches = [LayerCache(shape) for _ in range(reps)]
        alias = None
        for c in caches:
            alias = prefill_layer(c, wl, 0, ctx, plan, bt)
        o = torch.empty_like(q)
        max_ctx = int(ctx.max())
        for _ in range(warmup):
            for c in caches:
                c.decode(q, bt, ctx_g, max_ctx, out=o)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(calls * reps)]
        torch.cuda.synchronize()
        for i in range(calls):
            for r, c in enumerate(caches):
                a, b = ev[i * reps + r]
                a.record()
                c.decode(q, bt, ctx_g, max_ctx, out=o)
                b.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        nb = A.decode_bytes(ctx, wl.hq, wl.hkv)
        leg = {"batch": wl.batch, "q_heads": wl.hq, "kv_heads": wl.hkv, "replicas": reps,
               "calls": calls * reps, "call_ms": round(ms, 5), "bytes_per_call": nb,
               "gbs": round(nb / (ms * 1e-3) / 1e9, 2),
               "hbm_peak_frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "decode_tokens_per_s": round(wl.batch / (ms * 1e-3), 1)}
        if len(plan.sharing):
            ub = A.decode_bytes_unique(ctx, wl.hq, wl.hkv, alias)
            leg["bytes_per_call_logical"] = nb
            leg["bytes_per_call_unique"] = ub
            leg["gbs_unique"] = round(ub / (ms * 1e-3) / 1e9, 2)
        out[name] = leg
        print(f"[bench] {name}: {ms * 1000:.1f} us per call, {leg['gbs']:.0f} GB/s", file=sys.stderr,
              flush=True)
        del caches
        torch.cuda.empty_cache()
    return out


def cpu_baseline(t_attn=1.5, max_passes=50):
    """The CPU oracle on bounded samples of the workloads it validates, on the
    host's cores: the tiny case and the 3B-shaped layer in full, then layer 0
    of the 8B-shaped workload (its first 16 sequences), of the shared-prefix
    workload (first 8) and of the 70B-shaped workload (first 2). For each
    sample the oracle's quantizer (sequence_cache: every page of every
    sequence, plus the tails) is timed once, and its decode attention
    (dequantize the pages, then softmax attention in fp64) is repeated until
    about ``t_attn`` seconds; the two are reported separately, each in GB/s
    by the same byte accounting as the GPU path (quantize: fp16 K/V read,
    pages and tails written; attention: the decode bytes). ``value`` is the
    8B-shaped sample's attention rate. Nothing is extrapolated."""
    import oracle
    import threadpoolctl

    info = threadpoolctl.threadpool_info()
    blas_threads = max([i.get("num_threads", 1) for i in info] + [1])
    legs = {}
    for name, n_seqs in (("tiny", None), ("llama3.2-3b-layer", None), ("llama3.1-8b-decode", 16),
                         ("qwen2.5-7b-shared-prefix", 8), ("llama3-70b", 2)):
        wl = W.WORKLOADS[name]
        ctx = W.context_lengths(wl)[:n_seqs]
        mult = W.k_channel_multipliers(wl, 0)
        q = W.queries(wl, 0, "cpu").numpy()
        kvs = []
        for b in range(len(ctx)):
            k, v = W.sequence_kv(wl, 0, b, int(ctx[b]), "cpu", mult)
            kvs.append((k.numpy(), v.numpy()))
        t = time.perf_counter()
        caches = [oracle.sequence_cache(k, v) for k, v in kvs]
        t_q = time.perf_counter() - t
        del kvs
        full = (ctx // 16) * 16
        q_bytes = A.quantize_bytes(int(full.sum()), int((ctx - full).sum()), wl.hkv)
        d_bytes = A.decode_bytes(ctx, wl.hq, wl.hkv)
        passes, t_a = 0, 0.0
        while (t_a < t_attn or passes == 0) and passes < max_passes:
            t = time.perf_counter()
            for b, c in enumerate(caches):
                kh, vh = oracle.dequantized_sequence(c)
                oracle.decode_attention(q[b], kh, vh)
            t_a += time.perf_counter() - t
            passes += 1
        legs[name] = {
            "layer": 0, "sequences": int(len(ctx)), "ctx_sum": int(ctx.sum()),
            "quantize_s": round(t_q, 3), "quantize_gbs": round(q_bytes / t_q / 1e9, 4),
            "attention_passes": passes, "attention_s": round(t_a, 3),
            "attention_gbs": round(d_bytes * passes / t_a / 1e9, 4),
            "decode_tokens_per_s": round(len(ctx) * passes / t_a, 3),
        }
        print(f"[bench] cpu oracle {name}: quantize {legs[name]['quantize_gbs']} GB/s, "
              f"attention {legs[name]['attention_gbs']} GB/s", file=sys.stderr, flush=True)
    head = legs["llama3.1-8b-decode"]
    return {
        "value": head["attention_gbs"],
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": ("numpy oracle on the host: decode attention (dequantize + fp64 softmax "
                   "attention) of layer 0, first 16 sequences of llama3.1-8b-decode, repeated "
                   f"{head['attention_passes']} times ({head['attention_s']} s); quantizer and "
                   "the other configurations' samples under 'legs'"),
        "host_cores": len(os.sched_getaffinity(0)),
        "blas_threads": int(blas_threads),
        "legs": legs,
    }


def copy_ceiling(nbytes=1 << 30, reps=10):
    """Plain streaming kernel of known size (fp32 negation: reads and writes
    `nbytes` each) on the current stream: the measured bandwidth ceiling, and
    the dispatch whose FETCH_SIZE / WRITE_SIZE calibrate the decode counters."""
    import torch

    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.neg(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "avg_ms": round(ms, 5),
            "gbs": round(2 * nbytes / (ms * 1e-3) / 1e9, 2)}


def read_ceiling(reps=10):
    """What the decode kernels' load path sustains with nothing attached:
    s4kv_probe_read over 2 GiB in 4096-byte chunks taken in a random order,
    one wave per work-group, 8 per CU (the decode grid), one chunk in flight
    per wave; with and without the non-temporal policy the decode kernels use.
    Medians of `reps` calls timed with HIP events."""
    import torch
    from int4_kivi_quantized_amd import s4kv
    pool_bytes = 2 << 30
    pool = torch.empty(pool_bytes, dtype=torch.uint8, device="cuda")
    chunks = pool_bytes // 4096
    waves = 8 * torch.cuda.get_device_properties(0).multi_processor_count
    per = chunks // waves
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    ids = torch.randperm(chunks, generator=g, device="cuda", dtype=torch.int64)[:waves * per]
    ids = ids.to(torch.int32).contiguous()
    out = {"chunk_bytes": 4096, "order": "random", "waves": waves,
           "bytes_read": waves * per * 4096}
    for nt in (True, False):
        s4kv.s4kv_probe_read(pool, ids, per, waves, nt)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            s4kv.s4kv_probe_read(pool, ids, per, waves, nt)
            b.record()
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
        key = "non_temporal" if nt else "default_policy"
        out[key] = {"avg_ms": round(ms, 5), "gbs": round(out["bytes_read"] / (ms * 1e-3) / 1e9, 1)}
    del pool, ids
    torch.cuda.empty_cache()
    out["gbs"] = out["non_temporal"]["gbs"]
    return out


def graph_call_ms(fns, reps=10, rounds=15):
    """Per-call GPU time of each callable in `fns` ({name: launch one call}):
    `reps` consecutive calls captured in one HIP graph per name, the graphs
    replayed in turn `rounds` times (order alternating), each replay between
    two events on the current stream; the median over replays, divided by
    `reps`. This is the device time of the call without host launch gaps,
    as the headline's graph-replayed steps measure it."""
    import torch
    graphs = {}
    for name, fn in fns.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        graphs[name] = g
    torch.cuda.synchronize()
    for g in graphs.values():  # one untimed replay each
        g.replay()
    torch.cuda.synchronize()
    ev = {name: [] for name in fns}
    names = list(fns)
    for r in range(rounds):
        for name in (names if r % 2 == 0 else names[::-1]):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            graphs[name].replay()
            b.record()
            ev[name].append((a, b))
    torch.cuda.synchronize()
    res = {name: float(np.median([a.elapsed_time(b) for a, b in ev[name]])) / reps for name in fns}
    del graphs
    return res


def format_comparison(wl, calls=20, warmup=3):
    """The same decode over the four caches of this library on one layer of
    the workload: layer 0's cache built as int4 (s4kv_quantize_append), as
    2-bit KIVI (s4kv_kivi2_quantize_append), as fp16 (s4kv_fp16_append, the
    control path) and as FP8 E4M3
    (s4kv_fp8_append, per-KV-head scales calibrated on sequence 0: its
    largest magnitude over 448); then `calls` decode calls of each,
    interleaved, each timed with HIP events on the call's stream (medians,
    `eager_call_ms`), and the same calls replayed from HIP graphs
    (graph_call_ms: `call_ms`, the device time of a call, which the rates and
    ratios use), with each format's algorithmic bytes per call."""
    import torch
    from int4_kivi_quantized_amd import Shape
    from int4_kivi_quantized_amd.cache import Fp8LayerCache, Fp16LayerCache, Kivi2LayerCache, LayerCache

    ctx = W.context_lengths(wl)
    plan = W.plan_pages(wl, ctx)
    shape = Shape(wl.batch, wl.hq, wl.hkv, plan.num_pages, plan.max_pages)
    bt = torch.from_numpy(plan.block_table).cuda()
    mult = W.k_channel_multipliers(wl, 0)
    ks, vs = [], []
    for b in range(wl.batch):
        k, v = W.sequence_kv(wl, 0, b, int(ctx[b]), "cuda", mult)
        ks.append(k)
        vs.append(v)
    k_scale = ks[0].float().abs().amax(dim=(0, 2)) / 448.0
    v_scale = vs[0].float().abs().amax(dim=(0, 2)) / 448.0
    k_all, v_all = torch.cat(ks).contiguous(), torch.cat(vs).contiguous()
    del ks, vs
    cu = torch.tensor(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32), device="cuda")
    sl = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
    q = W.queries(wl, 0, "cuda")
    ctx_g = torch.from_numpy(ctx.astype(np.int32)).cuda()
    max_ctx = int(ctx.max())
    # all caches resident, calls interleaved, so no measurement sees a
    # different allocation history or clock state than the others
    caches = {"int4": LayerCache(shape), "kivi2": Kivi2LayerCache(shape),
              "fp16": Fp16LayerCache(shape), "fp8": Fp8LayerCache(shape, k_scale.cpu(), v_scale.cpu())}
    outs = {}
    for name, cache in caches.items():
        cache.append(k_all, v_all, cu, sl, int(ctx.max()), bt)
        outs[name] = torch.empty_like(q)
    del k_all, v_all
    for _ in range(warmup):
        for name, cache in caches.items():
            cache.decode(q, bt, ctx_g, max_ctx, out=outs[name])
    ev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                 for _ in range(calls)] for name in caches}
    torch.cuda.synchronize()
    for i in range(calls):
        for name, cache in caches.items():
            a, b = ev[name][i]
            a.record()
            cache.decode(q, bt, ctx_g, max_ctx, out=outs[name])
            b.record()
    torch.cuda.synchronize()
    eager = {name: float(np.median([a.elapsed_time(b) for a, b in ev[name]])) for name in caches}
    res = graph_call_ms({name: (lambda c=cache, o=outs[name]: c.decode(q, bt, ctx_g, max_ctx, out=o))
                         for name, cache in caches.items()})
    del caches, outs
    torch.cuda.empty_cache()
    nbytes = {"int4": A.decode_bytes(ctx, wl.hq, wl.hkv),
              "kivi2": A.decode_bytes(ctx, wl.hq, wl.hkv, A.K2_CHUNK_BYTES),
              "fp16": A.fp16_decode_bytes(ctx, wl.hq, wl.hkv),
              "fp8": A.fp8_decode_bytes(ctx, wl.hq, wl.hkv)}
    out = {"workload": f"{wl.name}, layer 0 (no append)", "calls": calls,
           "timing": "call_ms: graph-replayed (10 calls per graph, median of 15 replays); "
                     "eager_call_ms: eager launches between HIP events, median"}
    for name in ("int4", "kivi2", "fp16", "fp8"):
        gbs = nbytes[name] / (res[name] * 1e-3) / 1e9
        out[name] = {"call_ms": round(res[name], 5), "eager_call_ms": round(eager[name], 5),
                     "bytes_per_call": nbytes[name],
                     "gbs": round(gbs, 2), "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4)}
    out["int4_speedup_over_fp16"] = round(res["fp16"] / res["int4"], 4)
    out["int4_speedup_over_fp8"] = round(res["fp8"] / res["int4"], 4)
    out["kivi2_speedup_over_int4"] = round(res["int4"] / res["kivi2"], 4)
    out["kivi2_over_int4_time"] = round(res["kivi2"] / res["int4"], 4)
    out["kivi2_over_int4_time_eager"] = round(eager["kivi2"] / eager["int4"], 4)
    return out


def multiquery_leg(wl, max_q=4, calls=20, warmup=3):
    """Multi-query attention (speculative verify: max_q new tokens per
    sequence, already appended) against the one-token decode call, on layer 0
    of the workload's int4 cache: `calls` calls of each, interleaved, HIP-event
    medians (eager), and the same calls replayed from HIP graphs
    (graph_call_ms), which the reported call times and ratio use."""
    import torch
    from int4_kivi_quantized_amd import Shape
    from int4_kivi_quantized_amd.cache import LayerCache

    ctx = W.context_lengths(wl)
    plan = W.plan_pages(wl, ctx)
    shape = Shape(wl.batch, wl.hq, wl.hkv, plan.num_pages, plan.max_pages)
    bt = torch.from_numpy(plan.block_table).cuda()
    mult = W.k_channel_multipliers(wl, 0)
    cache = LayerCache(shape)
    ks, vs = [], []
    for b in range(wl.batch):
        k, v = W.sequence_kv(wl, 0, b, int(ctx[b]), "cuda", mult)
        ks.append(k)
        vs.append(v)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32), device="cuda")
    cache.append(torch.cat(ks).contiguous(), torch.cat(vs).contiguous(), cu,
                 torch.zeros(wl.batch, dtype=torch.int32, device="cuda"), int(ctx.max()), bt)
    del ks, vs
    ctx_g = torch.from_numpy(ctx.astype(np.int32)).cuda()
    max_ctx = int(ctx.max())
    q1 = W.queries(wl, 0, "cuda")
    t_counts = np.full(wl.batch, max_q)
    qm = W.normal_fp16((int(t_counts.sum()), wl.hq, wl.head_dim), 4242, "cuda")
    cu_q = torch.from_numpy(np.concatenate([[0], np.cumsum(t_counts)]).astype(np.int32)).cuda()
    out1, outm = torch.empty_like(q1), torch.empty_like(qm)
    run = {"decode": lambda: cache.decode(q1, bt, ctx_g, max_ctx, out=out1),
           "mq": lambda: cache.attend(qm, cu_q, max_q, bt, ctx_g, max_ctx, out=outm)}
    for _ in range(warmup):
        for f in run.values():
            f()
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(calls)] for k in run}
    torch.cuda.synchronize()
    for i in range(calls):
        for k, f in run.items():
            a, b = ev[k][i]
            a.record()
            f()
            b.record()
    torch.cuda.synchronize()
    eager = {k: float(np.median([a.elapsed_time(b) for a, b in ev[k]])) for k in run}
    ms = graph_call_ms(run)
    del cache, qm, outm, out1
    torch.cuda.empty_cache()
    mq_b = A.mq_bytes(ctx, t_counts, wl.hq, wl.hkv)
    return {
        "workload": f"{wl.name}, layer 0, {max_q} new tokens per sequence (causal)",
        "calls": calls,
        "mq_call_ms": round(ms["mq"], 5),
        "mq_bytes_per_call": mq_b,
        "mq_gbs": round(mq_b / (ms["mq"] * 1e-3) / 1e9, 2),
        "mq_query_tokens_per_s": round(int(t_counts.sum()) / (ms["mq"] * 1e-3), 1),
        "decode_call_ms": round(ms["decode"], 5),
        "mq_over_decode_time": round(ms["mq"] / ms["decode"], 4),
        "timing": "call times graph-replayed (10 calls per graph, median of 15 replays); "
                  "eager_*: eager launches between HIP events, median",
        "eager_mq_call_ms": round(eager["mq"], 5),
        "eager_decode_call_ms": round(eager["decode"], 5),
        "mq_over_decode_time_eager": round(eager["mq"] / eager["decode"], 4),
    }


def prefill_chunk_leg(wl, t_new=128, calls=10, warmup=2):
    """Chunked-prefill attention: t_new new tokens per sequence (already
    appended, the last t_new positions of each context) attend causally over
    layer 0 of the workload's int4 cache in one s4kv_paged_attention_mq call;
    with Hq/Hkv = 4 the tokens go to the matrix cores in column tiles of 4
    tokens. Reported: query tokens per second, and the attention's
    arithmetic rate: for each query token and query head, 2 * 128 flops for
    the logit and 2 * 128 for the output per visible cache position, against
    the fp16 dense matrix-core peak. HIP-event medians."""
    import torch
    from int4_kivi_quantized_amd import Shape
    from int4_kivi_quantized_amd.cache import LayerCache

    ctx = W.context_lengths(wl)
    plan = W.plan_pages(wl, ctx)
    shape = Shape(wl.batch, wl.hq, wl.hkv, plan.num_pages, plan.max_pages)
    bt = torch.from_numpy(plan.block_table).cuda()
    cache = LayerCache(shape)
    prefill_layer(cache, wl, 0, ctx, plan, bt)
    ctx_g = torch.from_numpy(ctx.astype(np.int32)).cuda()
    t_counts = np.full(wl.batch, t_new)
    qm = W.normal_fp16((int(t_counts.sum()), wl.hq, wl.head_dim), 4545, "cuda")
    cu_q = torch.from_numpy(np.concatenate([[0], np.cumsum(t_counts)]).astype(np.int32)).cuda()
    out = torch.empty_like(qm)
    max_ctx = int(ctx.max())
    for _ in range(warmup):
        cache.attend(qm, cu_q, t_new, bt, ctx_g, max_ctx, out=out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        cache.attend(qm, cu_q, t_new, bt, ctx_g, max_ctx, out=out)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    del cache, qm, out
    torch.cuda.empty_cache()
    # visible positions of token t (0-based among the new ones): ctx - t_new + t + 1
    visible = int(sum(t_new * (c - t_new) + t_new * (t_new + 1) // 2 for c in ctx))
    flops = 4.0 * wl.head_dim * wl.hq * visible
    tflops = flops / (ms * 1e-3) / 1e12
    gq = wl.hq // wl.hkv
    tile = max(1, 16 // gq)
    return {
        "workload": f"{wl.name}, layer 0, {t_new} new tokens per sequence (causal)",
        "calls": calls,
        "call_ms": round(ms, 4),
        "query_tokens_per_s": round(int(t_counts.sum()) / (ms * 1e-3), 1),
        "tokens_per_tile": tile,
        "tiles_per_sequence": -(-t_new // tile),
        "attention_tflops": round(tflops, 2),
        "mfma_fp16_peak_tflops": 2500.0,
        "mfma_peak_frac": round(tflops / 2500.0, 4),
    }


def load_traffic(digest):
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("sources_digest") != digest:
        return None
    return t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3.1-8b-decode", choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches only (by default each step is captured in a HIP "
                         "graph and the headline times graph replays; eager is reported beside it)")
    ap.add_argument("--separate-append", action="store_true",
                    help="time s4kv_quantize_append + s4kv_paged_decode per layer instead of the "
                         "fused s4kv_paged_decode_append")
    ap.add_argument("--layers", type=int, default=None,
                    help="profiling only: override the workload's layer count (the JSON "
                         "line then does not describe the named workload)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the int4 KIVI decode "
              "path here is a single-GPU kernel library with no collectives", file=sys.stderr)
        sys.exit(2)

    import torch
    from int4_kivi_quantized_amd import s4kv
    s4kv.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    wl = W.WORKLOADS[args.workload]
    if args.layers is not None:
        import dataclasses
        wl = dataclasses.replace(wl, layers=args.layers)
        args.no_secondary = True
    print(f"[bench] {wl.name}: layers={wl.layers} B={wl.batch} Hq={wl.hq} Hkv={wl.hkv} "
          f"steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    copy = copy_ceiling()
    print(f"[bench] copy ceiling {copy['gbs']:.0f} GB/s", file=sys.stderr, flush=True)
    rceil = read_ceiling()
    print(f"[bench] read ceiling {rceil['gbs']:.0f} GB/s (non-temporal), "
          f"{rceil['default_policy']['gbs']:.0f} GB/s (default policy)", file=sys.stderr, flush=True)
    fused = wl.append and not args.separate_append
    r = run_decode_bench(wl, args.steps, args.warmup, append=wl.append, fused=fused,
                         graph=not args.eager)
    del r["model"]
    torch.cuda.empty_cache()
    print(f"[bench] step {r['step_ms']:.3f} ms, {r['kv_gbs']:.0f} GB/s", file=sys.stderr, flush=True)

    if fused:
        # the timed region is one call per layer and nothing else
        call_ms = r["step_ms"] / wl.layers
        call_bytes = r["step_bytes"] / wl.layers
    else:
        call_ms, call_bytes = r["decode_launch_ms"], r["decode_launch_bytes"]
    call_gbs = call_bytes / (call_ms * 1e-3) / 1e9
    digest = _sources_digest(["paged_decode.hip", "internal.h"])
    traffic = load_traffic(digest)
    line = {
        "metric": METRIC,
        "value": round(r["kv_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 cache (u4 codes, f16 scale/zero), f16 q/o, f32 softmax",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "layers": wl.layers, "batch": wl.batch, "q_heads": wl.hq,
            "kv_heads": wl.hkv, "head_dim": wl.head_dim, "page": wl.page,
            "ctx": list(wl.ctx), "append_per_step": 1 if wl.append else 0,
            "layer_step": ("s4kv_paged_decode_append" if fused else
                           "s4kv_quantize_append + s4kv_paged_decode" if wl.append else
                           "s4kv_paged_decode"),
            "profiling_layer_override": args.layers,
            "launch": ("each step (all layers) captured in a HIP graph, timed as replays"
                       if r["graph"] else "eager launches"),
        },
        "eager_ms_per_step": round(r["eager_step_ms"], 4),
        "hbm_peak_frac": round(r["kv_gbs"] / HBM_PEAK_GBS, 4),
        "decode_tokens_per_s": round(r["tokens_per_s"], 1),
        "roofline": {
            "bound": "hbm",
            "kernel": ("one s4kv_paged_decode_append call on one layer (its two launches: decode "
                       "stream with the one-token append, split merge); the timed steps hold "
                       "nothing else, so its average duration is the HIP-event time of the timed "
                       "region (graph replays of whole steps) over the calls in it" if fused else
                       "one s4kv_paged_decode call on one layer (its two launches: decode stream, "
                       "split merge), timed with HIP events around each call on its stream"),
            "achieved": round(call_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(call_gbs / HBM_PEAK_GBS, 4),
            "avg_launch_ms": round(call_ms, 5),
            "bytes_per_launch": int(call_bytes),
            "traffic": (traffic or {}).get("hbm_bytes_per_launch"),
            "frac_of_copy_ceiling": round(call_gbs / copy["gbs"], 4),
            "frac_of_read_ceiling": round(call_gbs / rceil["gbs"], 4),
            "event_timed_call_ms": round(r["decode_launch_ms"], 5),
        },
        "copy_ceiling": copy,
        "read_ceiling": rceil,
    }
    if not args.no_secondary and wl.name != "llama3-70b":
        wl2 = W.WORKLOADS["llama3-70b"]
        print(f"[bench] secondary {wl2.name}", file=sys.stderr, flush=True)
        r2 = run_decode_bench(wl2, max(3, args.steps // 4), 1, append=False, graph=not args.eager)
        del r2["model"]
        torch.cuda.empty_cache()
        line["secondary"] = {
            "workload": wl2.name, "layers": wl2.layers, "batch": wl2.batch,
            "ms_per_step": round(r2["step_ms"], 4), "kv_gbs": round(r2["kv_gbs"], 2),
            "eager_ms_per_step": round(r2["eager_step_ms"], 4),
            "hbm_peak_frac": round(r2["kv_gbs"] / HBM_PEAK_GBS, 4),
            "decode_tokens_per_s": round(r2["tokens_per_s"], 1),
            "decode_launch_gbs": round(r2["decode_launch_gbs"], 2),
            "prefill_quantize_gbs": None if r2["prefill_gbs"] is None else round(r2["prefill_gbs"], 2),
            "prefill_ms_per_layer": round(r2["prefill_ms_per_layer"], 4),
        }
    if not args.no_secondary:
        print("[bench] format comparison (int4 / kivi2 / fp16 / fp8)", file=sys.stderr, flush=True)
        line["format_comparison"] = format_comparison(wl)
        torch.cuda.empty_cache()
        print("[bench] multi-query (verify) attention", file=sys.stderr, flush=True)
        line["multiquery"] = multiquery_leg(wl)
        torch.cuda.empty_cache()
        print("[bench] chunked prefill attention", file=sys.stderr, flush=True)
        line["prefill_chunk"] = prefill_chunk_leg(wl)
        torch.cuda.empty_cache()
    if not args.no_secondary:
        print("[bench] small configurations (tiny, 3B rotated, shared prefix)", file=sys.stderr,
              flush=True)
        line["small_configs"] = small_configs()
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
