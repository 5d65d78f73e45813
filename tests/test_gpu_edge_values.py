"""The quantizer's special cases and the ends of the fp16 range on the GPU,
through the C ABI, against the oracle.

Inputs come from tests/edge_values.py: every page carries K channels and V
tokens whose groups are uniform (scale +0), have a -0 minimum, underflow the
fp16 scale, force the clamp through a subnormal scale, sit on exact ties at
unit scale, or (``extreme``) reach +-65504. The rule is the asymmetric
min/scale code of the S4 KV product page (header paragraph, "Funktionsweise"
step 1) with round-half-to-even in fp32 and fp16 scale and zero.

* int4 and 2-bit pages built by bulk prefill and by ragged appends: codes,
  scale and zero bit patterns and tails bit-exact;
* the fused decode step completing edge pages: bit-exact pages and tails,
  output identical to append + decode;
* attention over the non-extreme edge pages within the parity bar, for the
  three column layouts of the decode kernel (G = 3, 8, 16);
* queries at the ends of the fp16 range against K pages of the largest fp16
  scale (8736 for int4, 43680 for 2 bits): one key dominates by a margin far
  beyond fp32 rounding, so the output is that key's value, and must be
  finite and equal to the oracle's; and queries of magnitude 2^-20, whose
  softmax is nearly uniform.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from int4_kivi_quantized_amd import Shape
from int4_kivi_quantized_amd.cache import Kivi2LayerCache, LayerCache
from tests import parity
from tests.edge_values import edge_pages, edge_tail

pytestmark = pytest.mark.gpu
F16 = np.float16


class EdgeCache:
    """One layer's cache (int4 or 2-bit) over a permuted pool, for explicit
    per-sequence fp16 K/V arrays."""

    def __init__(self, hq, hkv, ctx, bits, extra=0, seed=0):
        rng = np.random.default_rng(seed)
        self.ctx = np.asarray(ctx, dtype=np.int64)
        self.bits = bits
        need = (self.ctx + extra + 15) // 16
        self.max_pages = max(1, int(need.max()))
        self.num_pages = int(math.ceil(1.25 * need.sum())) + 1
        ids = rng.permutation(self.num_pages).astype(np.int32)
        bt = np.zeros((len(ctx), self.max_pages), dtype=np.int32)
        cur = 0
        for b, n in enumerate(need):
            bt[b, :n] = ids[cur:cur + n]
            cur += n
        self.bt_np = bt
        self.bt = torch.from_numpy(bt).cuda()
        self.shape = Shape(len(ctx), hq, hkv, self.num_pages, self.max_pages)
        self.cache = (LayerCache if bits == 4 else Kivi2LayerCache)(self.shape)
        self.cache.pages.fill_(0xAB)
        self.cache.tail_k.view(torch.int16).fill_(0x7E01)
        self.cache.tail_v.view(torch.int16).fill_(0x7E01)

    def append(self, pieces, starts):
        """pieces[b]: fp16 (k, v) [n_b, Hkv, 128] appended at position starts[b]."""
        counts = np.array([k.shape[0] for k, _ in pieces], dtype=np.int64)
        if counts.sum() == 0:
            return
        k = torch.from_numpy(np.concatenate([k for k, _ in pieces])).cuda().contiguous()
        v = torch.from_numpy(np.concatenate([v for _, v in pieces])).cuda().contiguous()
        cu = torch.tensor(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32), device="cuda")
        sl = torch.tensor(np.asarray(starts, dtype=np.int32), device="cuda")
        self.cache.append(k, v, cu, sl, int(counts.max()), self.bt)

    def check_pages(self, kvs, ctx=None):
        ctx = self.ctx if ctx is None else ctx
        view = self.cache.chunk_view()
        tk, tv = self.cache.tails()
        for b, (k, v) in enumerate(kvs):
            want = oracle.sequence_cache(k[:ctx[b]], v[:ctx[b]], self.bits)
            full = int(ctx[b]) // 16
            ids = torch.from_numpy(self.bt_np[b, :full].astype(np.int64)).cuda()
            got = view[ids].cpu().numpy()
            bad = parity.page_mismatches(got, want["pages"], self.bits)
            assert not bad, f"seq {b}: page fields differ from the oracle: {bad}"
            n = int(ctx[b]) % 16
            gk = tk[b, :, :n].permute(1, 0, 2).cpu().numpy()
            gv = tv[b, :, :n].permute(1, 0, 2).cpu().numpy()
            assert np.array_equal(gk.view(np.uint16), want["tail_k"].view(np.uint16)), f"seq {b}: tail K"
            assert np.array_equal(gv.view(np.uint16), want["tail_v"].view(np.uint16)), f"seq {b}: tail V"

    def decode(self, q, ctx=None):
        ctx = self.ctx if ctx is None else ctx
        cg = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).cuda()
        out = self.cache.decode(torch.from_numpy(q).cuda(), self.bt, cg, int(np.max(ctx)))
        torch.cuda.synchronize()
        return out.float().cpu().numpy()


def _sequences(hkv, extreme, seed):
    """Edge sequences: 6 pages + 7 tail tokens, 4 pages, 2 pages + 15 tail tokens."""
    kvs = []
    for i, (pages, tail) in enumerate(((6, 7), (4, 0), (2, 15))):
        k, v = edge_pages(pages, hkv, seed + 10 * i, extreme)
        tk, tv = edge_tail(tail, hkv, seed + 10 * i + 1)
        kvs.append((np.concatenate([k, tk]), np.concatenate([v, tv])))
    return kvs


def _oracle_out(kvs, q, bits):
    outs = []
    for b, (k, v) in enumerate(kvs):
        kh, vh = oracle.dequantized_sequence(oracle.sequence_cache(k, v, bits))
        outs.append(oracle.decode_attention(q[b], kh, vh))
    return np.stack(outs)


@pytest.mark.parametrize("bits", [4, 2])
def test_edge_pages_bitexact(bits):
    """Bulk prefill of half of each sequence, the rest in ragged appends."""
    print(f"[case] edge_pages_bitexact bits={bits}", flush=True)
    hkv = 2
    kvs = _sequences(hkv, extreme=True, seed=100 + bits)
    ctx = [k.shape[0] for k, _ in kvs]
    c = EdgeCache(4 * hkv, hkv, ctx, bits, seed=bits)
    pos = [n // 2 for n in ctx]
    c.append([(k[:p], v[:p]) for (k, v), p in zip(kvs, pos)], [0] * len(kvs))
    torch.cuda.synchronize()
    c.check_pages(kvs, np.array(pos))
    rng = np.random.default_rng(bits)
    while any(p < n for p, n in zip(pos, ctx)):
        step = [int(min(rng.integers(0, 7), n - p)) for p, n in zip(pos, ctx)]
        c.append([(k[p:p + s], v[p:p + s]) for (k, v), p, s in zip(kvs, pos, step)], pos)
        pos = [p + s for p, s in zip(pos, step)]
    torch.cuda.synchronize()
    c.check_pages(kvs)


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("g", [3, 8, 16])
def test_edge_pages_attention(bits, g):
    print(f"[case] edge_pages_attention bits={bits} g={g}", flush=True)
    hkv = 2
    kvs = _sequences(hkv, extreme=False, seed=200 + g)
    ctx = [k.shape[0] for k, _ in kvs]
    c = EdgeCache(g * hkv, hkv, ctx, bits, seed=g)
    c.append(kvs, [0] * len(kvs))
    c.check_pages(kvs)
    q = np.random.default_rng(g).standard_normal((len(kvs), g * hkv, 128)).astype(F16)
    got = c.decode(q)
    ok, max_abs, rel = parity.attention_ok(got, _oracle_out(kvs, q, bits))
    print(f"  max_abs={max_abs:.2e} rel_l2={rel:.2e}", flush=True)
    assert ok, (max_abs, rel)


@pytest.mark.parametrize("extreme", [True, False])
def test_edge_fused_completion(extreme):
    """Each sequence holds 15 tokens of its last page in the tail; the fused
    call appends the 16th, which completes an edge page (in the extreme case,
    pages with +-65504 groups)."""
    print(f"[case] edge_fused_completion extreme={extreme}", flush=True)
    hkv, g = 2, 4
    kvs = []
    for i, pages in enumerate((5, 1, 3, 8)):
        kvs.append(edge_pages(pages, hkv, 300 + 7 * i + extreme, extreme))
    ctx_full = np.array([k.shape[0] for k, _ in kvs])
    ctx0 = ctx_full - 1
    sep = EdgeCache(g * hkv, hkv, ctx0, 4, extra=1, seed=5)
    fus = EdgeCache(g * hkv, hkv, ctx0, 4, extra=1, seed=5)
    for c in (sep, fus):
        c.append([(k[:n], v[:n]) for (k, v), n in zip(kvs, ctx0)], [0] * len(kvs))
    q = np.random.default_rng(9).standard_normal((len(kvs), g * hkv, 128)).astype(F16)
    kn = torch.from_numpy(np.stack([k[-1] for k, _ in kvs])).cuda().contiguous()
    vn = torch.from_numpy(np.stack([v[-1] for _, v in kvs])).cuda().contiguous()
    qg = torch.from_numpy(q).cuda()
    ctx = torch.from_numpy(ctx_full.astype(np.int32)).cuda()
    cu = torch.arange(len(kvs) + 1, dtype=torch.int32, device="cuda")
    sep.cache.append(kn, vn, cu, torch.from_numpy(ctx0.astype(np.int32)).cuda(), 1, sep.bt)
    want = sep.cache.decode(qg, sep.bt, ctx, int(ctx_full.max()))
    got = fus.cache.decode_append(qg, kn, vn, fus.bt, ctx, int(ctx_full.max()))
    torch.cuda.synchronize()
    assert torch.equal(fus.cache.pages, sep.cache.pages), "pages differ from append + decode"
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "output differs"
    fus.check_pages(kvs, ctx_full)
    if not extreme:
        ok, max_abs, rel = parity.attention_ok(got.float().cpu().numpy(), _oracle_out(kvs, q, 4))
        print(f"  max_abs={max_abs:.2e} rel_l2={rel:.2e}", flush=True)
        assert ok, (max_abs, rel)


@pytest.mark.parametrize("bits", [4, 2])
def test_query_range_ends(bits):
    """K channel 5 of page 0 is -65504 except token 9 (+65504), the largest
    fp16 K scale; page 1's channel 5 is uniform -65504. Query heads put q_5 at
    +65504, at the largest value whose plain fp16 product with that scale
    fitted the former fixed pre-scale (119.9375 for int4, 23.984375 for 2
    bits), and at 1000, so key 9 dominates each of them; head 3 is
    N(0,1) * 2^-20 (near-uniform softmax). The output is compared with the
    oracle's under the parity bar, each head's outputs divided by max(1, its
    largest |O_ref|)."""
    print(f"[case] query_range_ends bits={bits}", flush=True)
    rng = np.random.default_rng(17)
    hkv, g = 1, 4
    k = (rng.standard_normal((40, hkv, 128)) * 0.5).astype(F16)
    v = rng.standard_normal((40, hkv, 128)).astype(F16)
    k[:16, 0, 5] = -65504.0
    k[9, 0, 5] = 65504.0
    k[16:32, 0, 5] = -65504.0
    v[9, 0, :64] = 60000.0               # the dominant key's value: large V scale too
    c = EdgeCache(g * hkv, hkv, [40], bits, seed=3)
    c.append([(k, v)], [0])
    c.check_pages([(k, v)])
    q = rng.standard_normal((1, g * hkv, 128)).astype(F16)
    q[0, 0, 5] = 65504.0
    q[0, 1, 5] = 119.9375 if bits == 4 else 23.984375
    q[0, 2, 5] = 1000.0
    q[0, 3] = (rng.standard_normal(128) * 2.0 ** -20).astype(F16)
    got = c.decode(q)
    assert np.isfinite(got).all(), "outputs must be finite over the whole fp16 query range"
    want = _oracle_out([(k, v)], q, bits)
    scale = np.maximum(1.0, np.abs(want).max(axis=-1, keepdims=True))
    ok, max_abs, rel = parity.attention_ok(got / scale, want / scale)
    print(f"  per-head scaled max_abs={max_abs:.2e} rel_l2={rel:.2e} "
          f"(scales {scale.ravel().round(1).tolist()})", flush=True)
    assert ok, (max_abs, rel)
