"""Build one layer's int4 cache on the GPU from a seeded workload, and compute
oracle references for chosen sequences. Test infrastructure."""

import math

import numpy as np
import torch

import oracle
import workload as W
from int4_kivi_quantized_amd import Shape
from int4_kivi_quantized_amd.cache import Fp8LayerCache, Fp16LayerCache, Kivi2LayerCache, LayerCache


def calibrated_fp8_scales(wl, layer=0, mult=None, device="cuda"):
    """Per-KV-head (k_scale, v_scale), fp32 [Hkv]: the largest magnitude of
    sequence 0 (prefix included) over 448, so that the calibration sample just
    fills the E4M3 range (the calibrated scales of the KV-quantization guide;
    other sequences may exceed it and saturate)."""
    n = int(W.context_lengths(wl)[0])
    k, v = W.sequence_kv(wl, layer, 0, n, device, mult)
    ks = k.float().abs().amax(dim=(0, 2)) / 448.0
    vs = v.float().abs().amax(dim=(0, 2)) / 448.0
    return ks.cpu().numpy().astype(np.float32), vs.cpu().numpy().astype(np.float32)


class LayerCase:
    """One layer of a workload: the GPU cache and everything needed to check it.

    kind: "int4" (s4kv_quantize_append / s4kv_paged_decode), "kivi2" (2-bit
    pages, s4kv_kivi2_*), "fp16" (the control cache, s4kv_fp16_*) or "fp8"
    (s4kv_fp8_*, with per-KV-head scales fp8_scales = (k_scale, v_scale);
    calibrated from sequence 0 by default)."""

    def __init__(self, wl, layer=0, ctx_lens=None, extra_tokens=0, pool_seed_salt=None, kind="int4",
                 fp8_scales=None):
        assert kind in ("int4", "kivi2", "fp16", "fp8")
        self.kind = kind
        self.fp16 = kind == "fp16"
        self.wl = wl
        self.layer = layer
        self.ctx = np.asarray(W.context_lengths(wl) if ctx_lens is None else ctx_lens, dtype=np.int64)
        self.plan = W.plan_pages(wl, self.ctx, extra_tokens)
        self.shape = Shape(wl.batch, wl.hq, wl.hkv, self.plan.num_pages, self.plan.max_pages)
        self.mult = W.k_channel_multipliers(wl, layer)
        if kind == "fp8":
            if fp8_scales is None:
                fp8_scales = calibrated_fp8_scales(wl, layer, self.mult)
            ks, vs = (np.broadcast_to(np.asarray(x, dtype=np.float32), (wl.hkv,)).copy()
                      for x in fp8_scales)
            self.k_scale, self.v_scale = ks, vs
            self.cache = Fp8LayerCache(self.shape, torch.from_numpy(ks), torch.from_numpy(vs))
        elif kind == "fp16":
            self.cache = Fp16LayerCache(self.shape)
        elif kind == "kivi2":
            self.cache = Kivi2LayerCache(self.shape)
        else:
            self.cache = LayerCache(self.shape)
        self.bits = 2 if kind == "kivi2" else 4
        self.block_table = torch.from_numpy(self.plan.block_table).cuda()
        self.ctx_gpu = torch.from_numpy(self.ctx.astype(np.int32)).cuda()
        self.q = W.queries(wl, layer, "cuda")

    # ------------------------------------------------------------- inputs
    def seq_kv(self, b, device="cuda"):
        return W.sequence_kv(self.wl, self.layer, b, int(self.ctx[b]), device, self.mult)

    def prefill(self):
        """Bulk prefill of every sequence through s4kv_quantize_append."""
        wl = self.wl
        alias = np.zeros(wl.batch, dtype=np.int64)
        if len(self.plan.sharing):
            share_pages = wl.shared_prefix // wl.page
            pk, pv = W.prefix_kv(wl, self.layer, "cuda", self.mult)
            pshape = Shape(1, wl.hq, wl.hkv, self.plan.num_pages, share_pages)
            scratch = LayerCache(Shape(1, wl.hq, wl.hkv, 1, share_pages))   # tails only
            bt = torch.from_numpy(self.plan.prefix_pages[None, :].copy()).cuda()
            cu = torch.tensor([0, wl.shared_prefix], dtype=torch.int32, device="cuda")
            sl = torch.zeros(1, dtype=torch.int32, device="cuda")
            from int4_kivi_quantized_amd import s4kv
            if self.kind == "fp16":
                s4kv.s4kv_fp16_append(pshape, pk.contiguous(), pv.contiguous(), cu, sl,
                                      wl.shared_prefix, bt, self.cache.pages)
            elif self.kind == "fp8":
                s4kv.s4kv_fp8_append(pshape, pk.contiguous(), pv.contiguous(), cu, sl,
                                     wl.shared_prefix, bt, self.cache.k_scale, self.cache.v_scale,
                                     self.cache.pages)
            elif self.kind == "kivi2":
                s4kv.s4kv_kivi2_quantize_append(pshape, pk.contiguous(), pv.contiguous(), cu, sl,
                                                wl.shared_prefix, bt, self.cache.pages,
                                                scratch.tail_k, scratch.tail_v)
            else:
                s4kv.s4kv_quantize_append(pshape, pk.contiguous(), pv.contiguous(), cu, sl,
                                          wl.shared_prefix, bt, self.cache.pages, scratch.tail_k,
                                          scratch.tail_v)
            for b in self.plan.sharing:
                alias[b] = min(share_pages, int(self.ctx[b]) // wl.page)
        ks, vs, starts, counts = [], [], [], []
        for b in range(wl.batch):
            k, v = self.seq_kv(b)
            st = int(alias[b]) * wl.page
            ks.append(k[st:])
            vs.append(v[st:])
            starts.append(st)
            counts.append(int(self.ctx[b]) - st)
        k_all = torch.cat(ks).contiguous()
        v_all = torch.cat(vs).contiguous()
        del ks, vs
        cu = torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device="cuda")
        sl = torch.tensor(np.asarray(starts, dtype=np.int32), device="cuda")
        self.cache.append(k_all, v_all, cu, sl, max(counts), self.block_table)
        torch.cuda.synchronize()

    def decode(self, max_ctx=None):
        if max_ctx is None:
            max_ctx = int(self.ctx.max())
        out = self.cache.decode(self.q, self.block_table, self.ctx_gpu, max_ctx)
        torch.cuda.synchronize()
        return out

    # ------------------------------------------------------------- oracle side
    def oracle_seq(self, b):
        k, v = self.seq_kv(b)
        return oracle.sequence_cache(k.cpu().numpy(), v.cpu().numpy(), self.bits)

    def oracle_out(self, b, heads=None):
        c = self.oracle_seq(b)
        kh, vh = oracle.dequantized_sequence(c)
        q = self.q[b].cpu().numpy()
        if heads is not None:
            # evaluate only the chosen query heads (each reads KV head j // G)
            g = self.wl.group
            out = np.zeros((self.wl.hq, self.wl.head_dim))
            for j in heads:
                h = j // g
                out[j] = oracle.decode_attention(q[j:j + 1], kh[:, h:h + 1], vh[:, h:h + 1])[0]
            return out
        return oracle.decode_attention(q, kh, vh)

    def gpu_chunks(self, b):
        """uint8 [full_b, Hkv, stride] of sequence b's full pages (int4 or 2-bit pool)."""
        full = int(self.ctx[b]) // self.wl.page
        ids = self.plan.block_table[b, :full]
        return self.cache.chunk_view()[torch.from_numpy(ids.astype(np.int64)).cuda()].cpu().numpy()

    def gpu_fp16_pages(self, b):
        """fp16 [pages_b, Hkv, 4096] of sequence b's pages (fp16 cache)."""
        n = -(-int(self.ctx[b]) // self.wl.page)
        ids = self.plan.block_table[b, :n]
        return self.cache.chunk_view()[torch.from_numpy(ids.astype(np.int64)).cuda()].cpu().numpy()

    def gpu_fp8_pages(self, b):
        """uint8 [pages_b, Hkv, 4096] of sequence b's pages (FP8 cache)."""
        n = -(-int(self.ctx[b]) // self.wl.page)
        ids = self.plan.block_table[b, :n]
        return self.cache.chunk_view()[torch.from_numpy(ids.astype(np.int64)).cuda()].cpu().numpy()

    def gpu_tail(self, b):
        tk, tv = self.cache.tails()
        n = int(self.ctx[b]) % self.wl.page
        return tk[b, :, :n].permute(1, 0, 2).cpu().numpy(), tv[b, :, :n].permute(1, 0, 2).cpu().numpy()


def default_scale(d=128):
    return 1.0 / math.sqrt(d)
