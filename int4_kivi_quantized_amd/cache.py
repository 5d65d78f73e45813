"""Device buffers of one layer's int4 KIVI cache, allocated with torch.

A convenience over the C ABI for Python callers: it owns the page pool, the
two fp16 tails and the decode workspace of one layer and forwards every call
to libs4kv.so. The block table and context lengths stay with the caller (they
are shared by all layers of a model).
"""

import math

import torch

from . import s4kv


class LayerCache:
    def __init__(self, shape, device="cuda"):
        if s4kv.s4kv_validate(shape) != s4kv.S4KV_OK:
            raise s4kv.S4KVError(s4kv.s4kv_validate(shape), "LayerCache")
        self.shape = shape
        self.device = torch.device(device)
        self.pages = torch.zeros(s4kv.s4kv_pool_bytes(shape), dtype=torch.uint8, device=self.device)
        n_tail = s4kv.s4kv_tail_bytes(shape) // 2
        self.tail_k = torch.zeros(n_tail, dtype=torch.float16, device=self.device)
        self.tail_v = torch.zeros(n_tail, dtype=torch.float16, device=self.device)
        self._ws = None
        self._ws_ctx = 0

    def workspace(self, max_ctx):
        need = s4kv.s4kv_decode_workspace_bytes(self.shape, max_ctx)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def append(self, k, v, cu_new, slot, max_new, block_table, stream=None):
        s4kv.s4kv_quantize_append(self.shape, k, v, cu_new, slot, max_new, block_table,
                                  self.pages, self.tail_k, self.tail_v, stream)

    def decode(self, q, block_table, ctx_lens, max_ctx, sm_scale=None, out=None, stream=None):
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(self.shape.head_dim)
        if out is None:
            out = torch.empty_like(q)
        s4kv.s4kv_paged_decode(self.shape, q, self.pages, self.tail_k, self.tail_v, block_table,
                               ctx_lens, max_ctx, sm_scale, out, self.workspace(max_ctx), stream)
        return out

    def decode_append(self, q, k_new, v_new, block_table, ctx_lens, max_ctx, sm_scale=None,
                      out=None, stream=None):
        """Append one token per sequence (ctx_lens already count it) and decode."""
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(self.shape.head_dim)
        if out is None:
            out = torch.empty_like(q)
        s4kv.s4kv_paged_decode_append(self.shape, q, k_new, v_new, self.pages, self.tail_k,
                                      self.tail_v, block_table, ctx_lens, max_ctx, sm_scale, out,
                                      self.workspace(max_ctx), stream)
        return out

    def mq_workspace(self, max_ctx, max_q):
        need = s4kv.s4kv_mq_workspace_bytes(self.shape, max_ctx, max_q)
        if need == 0:
            raise s4kv.S4KVError(s4kv.S4KV_ERR_UNSUPPORTED, "mq_workspace")
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def attend(self, q, cu_q, max_q, block_table, ctx_lens, max_ctx, sm_scale=None, out=None,
               stream=None):
        """Multi-query attention of q fp16 [total_q, Hq, 128] (rows of sequence b:
        cu_q[b] .. cu_q[b+1]-1, the last ones in the cache) over this layer."""
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(self.shape.head_dim)
        if out is None:
            out = torch.empty_like(q)
        s4kv.s4kv_paged_attention_mq(self.shape, q, cu_q, max_q, self.pages, self.tail_k,
                                     self.tail_v, block_table, ctx_lens, max_ctx, sm_scale, out,
                                     self.mq_workspace(max_ctx, max_q), stream)
        return out

    def chunk_view(self):
        """uint8 [num_pages, Hkv, CHUNK_STRIDE] view of the pool."""
        return self.pages.view(self.shape.num_pages, self.shape.num_kv_heads, s4kv.CHUNK_STRIDE)

    def tails(self):
        """(tail_k, tail_v) as fp16 [B, Hkv, 16, 128] views."""
        s = self.shape
        dims = (s.num_seqs, s.num_kv_heads, s.page_size, s.head_dim)
        return self.tail_k.view(*dims), self.tail_v.view(*dims)


class Kivi2LayerCache(LayerCache):
    """One layer's 2-bit KIVI cache: the int4 cache's tails and workspace with a
    2-bit page pool and the s4kv_kivi2_* entry points."""

    def __init__(self, shape, device="cuda"):
        super().__init__(shape, device)
        self.pages = torch.zeros(s4kv.s4kv_kivi2_pool_bytes(shape), dtype=torch.uint8,
                                 device=self.device)

    def append(self, k, v, cu_new, slot, max_new, block_table, stream=None):
        s4kv.s4kv_kivi2_quantize_append(self.shape, k, v, cu_new, slot, max_new, block_table,
                                        self.pages, self.tail_k, self.tail_v, stream)

    def decode(self, q, block_table, ctx_lens, max_ctx, sm_scale=None, out=None, stream=None):
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(self.shape.head_dim)
        if out is None:
            out = torch.empty_like(q)
        s4kv.s4kv_kivi2_paged_decode(self.shape, q, self.pages, self.tail_k, self.tail_v,
                                     block_table, ctx_lens, max_ctx, sm_scale, out,
                                     self.workspace(max_ctx), stream)
        return out

    def attend(self, *args, **kwargs):
        raise NotImplementedError("multi-query attention runs over int4 pages only")

    def chunk_view(self):
        """uint8 [num_pages, Hkv, 1664] view of the pool."""
        return self.pages.view(self.shape.num_pages, self.shape.num_kv_heads,
                               s4kv.K2_CHUNK_STRIDE)


class Fp16LayerCache:
    """One layer's fp16 paged cache (the control path): pool and workspace."""

    def __init__(self, shape, device="cuda"):
        if s4kv.s4kv_validate(shape) != s4kv.S4KV_OK:
            raise s4kv.S4KVError(s4kv.s4kv_validate(shape), "Fp16LayerCache")
        self.shape = shape
        self.device = torch.device(device)
        self.pages = torch.zeros(s4kv.s4kv_fp16_pool_bytes(shape) // 2, dtype=torch.float16,
                                 device=self.device)
        self._ws = None

    def workspace(self, max_ctx):
        need = s4kv.s4kv_decode_workspace_bytes(self.shape, max_ctx)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def append(self, k, v, cu_new, slot, max_new, block_table, stream=None):
        s4kv.s4kv_fp16_append(self.shape, k, v, cu_new, slot, max_new, block_table, self.pages,
                              stream)

    def decode(self, q, block_table, ctx_lens, max_ctx, sm_scale=None, out=None, stream=None):
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(self.shape.head_dim)
        if out is None:
            out = torch.empty_like(q)
        s4kv.s4kv_fp16_paged_decode(self.shape, q, self.pages, block_table, ctx_lens, max_ctx,
                                    sm_scale, out, self.workspace(max_ctx), stream)
        return out

    def chunk_view(self):
        """fp16 [num_pages, Hkv, 4096] view of the pool."""
        return self.pages.view(self.shape.num_pages, self.shape.num_kv_heads,
                               s4kv.F16_CHUNK_BYTES // 2)


class Fp8LayerCache:
    """One layer's FP8 (E4M3) paged cache: pool, per-KV-head scales and workspace.

    k_scale / v_scale: fp32 [Hkv] (or scalars, broadcast), fixed for the cache's
    lifetime; 1.0 is the uncalibrated default."""

    def __init__(self, shape, k_scale=1.0, v_scale=1.0, device="cuda"):
        if s4kv.s4kv_validate(shape) != s4kv.S4KV_OK:
            raise s4kv.S4KVError(s4kv.s4kv_validate(shape), "Fp8LayerCache")
        self.shape = shape
        self.device = torch.device(device)
        self.pages = torch.zeros(s4kv.s4kv_fp8_pool_bytes(shape), dtype=torch.uint8,
                                 device=self.device)
        h = shape.num_kv_heads
        self.k_scale = torch.as_tensor(k_scale, dtype=torch.float32).expand(h).contiguous().to(self.device)
        self.v_scale = torch.as_tensor(v_scale, dtype=torch.float32).expand(h).contiguous().to(self.device)
        self._ws = None

    def workspace(self, max_ctx):
        need = s4kv.s4kv_decode_workspace_bytes(self.shape, max_ctx)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def append(self, k, v, cu_new, slot, max_new, block_table, stream=None):
        s4kv.s4kv_fp8_append(self.shape, k, v, cu_new, slot, max_new, block_table, self.k_scale,
                             self.v_scale, self.pages, stream)

    def decode(self, q, block_table, ctx_lens, max_ctx, sm_scale=None, out=None, stream=None):
        if sm_scale is None:
            sm_scale = 1.0 / math.sqrt(self.shape.head_dim)
        if out is None:
            out = torch.empty_like(q)
        s4kv.s4kv_fp8_paged_decode(self.shape, q, self.pages, block_table, ctx_lens, max_ctx,
                                   sm_scale, self.k_scale, self.v_scale, out,
                                   self.workspace(max_ctx), stream)
        return out

    def chunk_view(self):
        """uint8 [num_pages, Hkv, 4096] view of the pool."""
        return self.pages.view(self.shape.num_pages, self.shape.num_kv_heads,
                               s4kv.FP8_CHUNK_BYTES)
