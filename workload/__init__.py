"""Seeded synthetic workloads for the int4 KIVI paged cache.

This module only draws inputs: random fp16 K/V/Q tensors, context lengths,
outlier channels, block tables over a permuted page pool and shared-prefix
aliasing. It holds none of the quantizer's or attention's arithmetic, so both
the CPU oracle side and the GPU side can take their inputs from it.

Workload shapes follow the model families named on the S4 KV product page
("Lieferumfang": Qwen2.5 and Llama-3 families, head_dim 128) and the page size
of 16 tokens from the PagedAttention explainers (polaris7.io signal page,
"Wichtigste Kernpunkte & Evidenz"). The draws (distributions, outlier
fraction, context-length mix, pool over-provisioning, shared prefix) are this
project's synthetic stand-ins for real traffic; the recipe is spelled out in
each field below.
"""

from dataclasses import dataclass, field
import math

import numpy as np

HEAD_DIM = 128
PAGE = 16


@dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    hq: int
    hkv: int
    ctx: tuple                 # ("fixed", n) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    k_outliers: tuple          # ("count", n, lo, hi) | ("frac", f, lo, hi): K channels scaled by U[lo, hi]
    shared_prefix: int = 0     # tokens whose pages half of the sequences share
    pool_factor: float = 1.25  # physical pages = ceil(factor * distinct pages needed)
    append: bool = False       # a step appends one token per sequence before decoding
    seed: int = 0
    head_dim: int = HEAD_DIM
    page: int = PAGE

    @property
    def group(self):
        return self.hq // self.hkv


WORKLOADS = {
    # 1 sequence, 1 layer, 4 query heads / 1 KV head, 256 tokens; 4 K channels x10
    "tiny": Workload("tiny", 1, 1, 4, 1, ("fixed", 256), ("count", 4, 10.0, 10.0),
                     pool_factor=1.0),
    # Llama-3.2-3B-shaped layer: 24/8 heads, batch 32, ctx U[512, 4096]
    "llama3.2-3b-layer": Workload("llama3.2-3b-layer", 1, 32, 24, 8, ("uniform", 512, 4096),
                                  ("frac", 0.02, 8.0, 20.0), seed=1),
    # Llama-3.1-8B-shaped decode: 32 layers, 32/8 heads, batch 128, ctx U[2048, 8192],
    # one appended token per sequence per step
    "llama3.1-8b-decode": Workload("llama3.1-8b-decode", 32, 128, 32, 8, ("uniform", 2048, 8192),
                                   ("frac", 0.02, 8.0, 20.0), append=True, seed=2),
    # Qwen2.5-7B-shaped layer: 28/4 heads, batch 64, ctx log-uniform [1024, 32768],
    # half the sequences share the pages of a 2048-token prefix
    "qwen2.5-7b-shared-prefix": Workload("qwen2.5-7b-shared-prefix", 1, 64, 28, 4,
                                         ("loguniform", 1024, 32768), ("frac", 0.02, 8.0, 20.0),
                                         shared_prefix=2048, seed=3),
    # Llama-3-70B-shaped: 80 layers, 64/8 heads, batch 16, 32768-token contexts built by
    # one bulk prefill per layer
    "llama3-70b": Workload("llama3-70b", 80, 16, 64, 8, ("fixed", 32768), ("frac", 0.02, 8.0, 20.0),
                           seed=4),
}


def rng_for(wl, *salt):
    """numpy Generator seeded by the workload seed and a salt tuple."""
    return np.random.default_rng([wl.seed, *[int(s) for s in salt]])


def context_lengths(wl):
    r = rng_for(wl, 1)
    kind = wl.ctx[0]
    if kind == "fixed":
        return np.full(wl.batch, wl.ctx[1], dtype=np.int64)
    lo, hi = wl.ctx[1], wl.ctx[2]
    if kind == "uniform":
        return r.integers(lo, hi + 1, size=wl.batch).astype(np.int64)
    if kind == "loguniform":
        x = np.exp(r.uniform(math.log(lo), math.log(hi), size=wl.batch))
        return np.clip(np.round(x), lo, hi).astype(np.int64)
    raise ValueError(kind)


def sharing_sequences(wl):
    """Indices of the sequences whose first ``shared_prefix`` tokens are shared."""
    if not wl.shared_prefix:
        return np.zeros(0, dtype=np.int64)
    r = rng_for(wl, 2)
    return np.sort(r.choice(wl.batch, size=wl.batch // 2, replace=False)).astype(np.int64)


def k_channel_multipliers(wl, layer):
    """float32 [Hkv, D]: 1 for ordinary K channels, U[lo, hi] for outlier channels."""
    r = rng_for(wl, 3, layer)
    kind, a, lo, hi = wl.k_outliers
    mult = np.ones((wl.hkv, wl.head_dim), dtype=np.float32)
    n = int(a) if kind == "count" else max(1, int(round(a * wl.head_dim)))
    for h in range(wl.hkv):
        ch = r.choice(wl.head_dim, size=n, replace=False)
        mult[h, ch] = r.uniform(lo, hi, size=n).astype(np.float32)
    return mult


@dataclass
class PagePlan:
    """Logical -> physical page mapping for one workload (shared by all layers)."""
    num_pages: int
    block_table: np.ndarray          # int32 [B, max_pages]; unused entries are 0
    max_pages: int
    prefix_pages: np.ndarray         # int32 [shared_prefix // 16] physical ids of the shared prefix
    sharing: np.ndarray              # sequence indices that alias the prefix pages
    distinct_pages: int


def plan_pages(wl, ctx_lens, extra_tokens=0):
    """Build block tables over a randomly permuted pool of ``pool_factor`` x demand.

    ``extra_tokens`` reserves room for tokens appended later (decode steps).
    Sequences in :func:`sharing_sequences` map their first ``shared_prefix //
    16`` logical pages to one common set of physical pages.
    """
    r = rng_for(wl, 4)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    sharing = sharing_sequences(wl)
    share_pages = wl.shared_prefix // wl.page
    need = (ctx_lens + extra_tokens + wl.page - 1) // wl.page
    max_pages = int(need.max())
    private = need.copy()
    # a sharing sequence aliases only the prefix pages it has filled; its
    # partial page (if any) is private, so later appends never write a shared page
    alias = np.zeros(wl.batch, dtype=np.int64)
    for b in sharing:
        alias[b] = min(share_pages, int(ctx_lens[b]) // wl.page)
        private[b] = need[b] - alias[b]
    distinct = int(private.sum()) + (share_pages if len(sharing) else 0)
    num_pages = max(1, int(math.ceil(wl.pool_factor * distinct)))
    ids = r.permutation(num_pages).astype(np.int32)
    cursor = 0
    prefix_ids = np.zeros(0, dtype=np.int32)
    if len(sharing):
        prefix_ids = ids[:share_pages].copy()
        cursor = share_pages
    bt = np.zeros((wl.batch, max_pages), dtype=np.int32)
    shared_set = set(int(b) for b in sharing)
    for b in range(wl.batch):
        start = 0
        if b in shared_set:
            k = int(alias[b])
            bt[b, :k] = prefix_ids[:k]
            start = k
        n = int(need[b]) - start
        bt[b, start:start + n] = ids[cursor:cursor + n]
        cursor += n
    return PagePlan(num_pages, bt, max_pages, prefix_ids, sharing, distinct)


def _torch():
    import torch
    return torch


def normal_fp16(shape, seed, device="cpu"):
    """fp16 N(0,1) tensor from a torch generator seeded with ``seed`` on ``device``."""
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.float16)


def layer_seed(wl, layer, what, seq=0):
    return (wl.seed * 1_000_003 + layer * 10_007 + seq * 101 + {"k": 1, "v": 2, "q": 3, "pk": 4, "pv": 5, "nk": 6, "nv": 7}[what]) & 0x7FFFFFFF


def sequence_kv(wl, layer, b, ctx, device="cpu", mult=None):
    """fp16 K, V [ctx, Hkv, D] of sequence ``b`` in ``layer``.

    K is N(0,1) times the layer's channel multipliers; V is N(0,1). Sequences
    that share the prefix take its first ``shared_prefix`` tokens from
    :func:`prefix_kv`.
    """
    torch = _torch()
    if mult is None:
        mult = k_channel_multipliers(wl, layer)
    m = torch.from_numpy(mult).to(device)
    k = (normal_fp16((ctx, wl.hkv, wl.head_dim), layer_seed(wl, layer, "k", b), device).float() * m).half()
    v = normal_fp16((ctx, wl.hkv, wl.head_dim), layer_seed(wl, layer, "v", b), device)
    if wl.shared_prefix and b in set(int(x) for x in sharing_sequences(wl)):
        pk, pv = prefix_kv(wl, layer, device, mult)
        n = min(ctx, wl.shared_prefix)
        k[:n] = pk[:n]
        v[:n] = pv[:n]
    return k, v


def prefix_kv(wl, layer, device="cpu", mult=None):
    torch = _torch()
    if mult is None:
        mult = k_channel_multipliers(wl, layer)
    m = torch.from_numpy(mult).to(device)
    n = wl.shared_prefix
    k = (normal_fp16((n, wl.hkv, wl.head_dim), layer_seed(wl, layer, "pk"), device).float() * m).half()
    v = normal_fp16((n, wl.hkv, wl.head_dim), layer_seed(wl, layer, "pv"), device)
    return k, v


def queries(wl, layer, device="cpu"):
    """fp16 Q [B, Hq, D] ~ N(0,1)."""
    return normal_fp16((wl.batch, wl.hq, wl.head_dim), layer_seed(wl, layer, "q"), device)


def new_tokens(wl, layer, step, device="cpu", mult=None):
    """fp16 K, V [B, Hkv, D] appended at decode ``step`` (same distributions)."""
    torch = _torch()
    if mult is None:
        mult = k_channel_multipliers(wl, layer)
    m = torch.from_numpy(mult).to(device)
    shape = (wl.batch, wl.hkv, wl.head_dim)
    k = (normal_fp16(shape, layer_seed(wl, layer, "nk", step), device).float() * m).half()
    v = normal_fp16(shape, layer_seed(wl, layer, "nv", step), device)
    return k, v
