"""FP8 (E4M3) cache vs the oracle, through the C ABI (libs4kv.so).

Append: every defined token slot of the FP8 pool holds the oracle's E4M3 code
of the input under the KV head's scale, bit for bit (read back through the
page format of include/s4kv.h). The pool is filled with 0x7F bytes (E4M3 NaN)
first, so a slot the kernels wrongly read, or an undefined slot of a partial
page that reached the arithmetic, shows up in the outputs. Decode: attention
over the oracle's dequantized K and V within 2e-3 max-abs and 1e-3 relative L2
(plain softmax attention in float64). The code read-out test pins the decode
kernel's conversion of every finite code exactly.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
import workload as W
from int4_kivi_quantized_amd import Shape
from int4_kivi_quantized_amd.cache import Fp8LayerCache
from tests import layout, parity
from tests.gpu_harness import LayerCase

pytestmark = pytest.mark.gpu

NAN_BYTE = 0x7F


def _print_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _case(wl, **kw):
    case = LayerCase(wl, kind="fp8", **kw)
    case.cache.pages.fill_(NAN_BYTE)
    case.prefill()
    return case


def _oracle_codes(case, b):
    k, v = case.seq_kv(b)
    return ofp8.fp8_sequence(k.cpu().numpy(), v.cpu().numpy(), case.k_scale, case.v_scale)


def _check_pages(case, seqs):
    for b in seqs:
        kc, vc = _oracle_codes(case, b)                    # [ctx, Hkv, 128]
        gk, gv = layout.read_fp8_chunks(case.gpu_fp8_pages(b))   # [pages, Hkv, 16, 128]
        n = int(case.ctx[b])
        for p in range(gk.shape[0]):
            t0, t1 = 16 * p, min(n, 16 * p + 16)
            want_k = kc[t0:t1].transpose(1, 0, 2)          # [Hkv, tokens, 128]
            want_v = vc[t0:t1].transpose(1, 0, 2)
            assert np.array_equal(gk[p, :, :t1 - t0], want_k), f"seq {b} page {p}: K codes differ"
            assert np.array_equal(gv[p, :, :t1 - t0], want_v), f"seq {b} page {p}: V codes differ"


def _oracle_out(case, b):
    kc, vc = _oracle_codes(case, b)
    kh, vh = ofp8.fp8_dequantized(kc, vc, case.k_scale, case.v_scale)
    return oracle.decode_attention(case.q[b].cpu().numpy(), kh, vh)


def _check_decode(case, seqs):
    out = case.decode().float().cpu().numpy()
    got = np.concatenate([out[b] for b in seqs])
    want = np.concatenate([_oracle_out(case, b) for b in seqs])
    assert np.isfinite(got).all(), "non-finite output"
    ok, max_abs, rel = parity.attention_ok(got, want)
    print(f"  fp8 decode max_abs={max_abs:.2e} rel_l2={rel:.2e} outputs={len(got)}", flush=True)
    assert ok, f"attention out of tolerance: max_abs={max_abs:.3e} rel_l2={rel:.3e}"


@pytest.mark.parametrize("v_scale", [1.0, 0.125, 3.0])
def test_fp8_code_readout(v_scale):
    """Sequences of one token: the output is that token's V, value(code) x
    v_scale, exactly. Pages written from the host in the documented format;
    every finite code appears once, undefined slots hold NaN codes."""
    _print_case("fp8_code_readout", v_scale=v_scale)
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)   # 254
    nseq = 2
    vcodes = np.zeros((nseq, 128), dtype=np.uint8)
    vcodes.reshape(-1)[:len(codes)] = codes
    vcodes.reshape(-1)[len(codes):] = 0x38                                          # 1.0
    shape = Shape(nseq, 1, 1, nseq, 1)
    cache = Fp8LayerCache(shape, 0.5, v_scale)
    raw = np.empty((nseq, layout.FP8_CHUNK_BYTES), dtype=np.uint8)
    for b in range(nseq):
        kc = np.full((16, 128), NAN_BYTE, dtype=np.uint8)
        vc = np.full((16, 128), NAN_BYTE, dtype=np.uint8)
        kc[0] = 0x30                                                               # 0.5
        vc[0] = vcodes[b]
        raw[b] = layout.write_fp8_chunk(kc, vc)
    cache.pages.copy_(torch.from_numpy(raw.reshape(-1)).cuda())
    q = torch.ones((nseq, 1, 128), dtype=torch.float16, device="cuda")
    bt = torch.arange(nseq, dtype=torch.int32, device="cuda").view(nseq, 1)
    ctx = torch.ones(nseq, dtype=torch.int32, device="cuda")
    out = cache.decode(q, bt, ctx, 1)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()[:, 0]
    want = (ofp8.e4m3_value(vcodes) * v_scale).astype(np.float16).astype(np.float32)
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, f"codes {vcodes[bad][:8]} read {got[bad][:8]} want {want[bad][:8]}"


@pytest.mark.parametrize("name", ["tiny", "llama3.2-3b-layer"])
def test_fp8_pages_and_decode(name):
    _print_case("fp8_pages_and_decode", workload=name)
    case = _case(W.WORKLOADS[name])
    _check_pages(case, range(case.wl.batch))
    _check_decode(case, range(case.wl.batch))


@pytest.mark.parametrize("g", [1, 3, 4, 7, 8, 16])
def test_fp8_edge_contexts(g):
    _print_case("fp8_edge_contexts", group=g)
    ctx = np.array([1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257, 1000, 4111], dtype=np.int64)
    hkv = 2
    wl = W.Workload(f"f8-edge-g{g}", 1, len(ctx), g * hkv, hkv, ("fixed", 1),
                    ("frac", 0.02, 8.0, 20.0), seed=70 + g)
    case = _case(wl, ctx_lens=ctx)
    _check_pages(case, range(wl.batch))
    _check_decode(case, range(wl.batch))


@pytest.mark.parametrize("scales", ["unit", "tight"])
def test_fp8_scales_and_saturation(scales):
    """Uncalibrated scales (1.0: small values fall into the subnormal codes)
    and scales far too small (most K outliers and V tails saturate at 448):
    codes stay bit-exact and attention follows the oracle over the same codes."""
    _print_case("fp8_scales_and_saturation", scales=scales)
    wl = W.WORKLOADS["llama3.2-3b-layer"]
    if scales == "unit":
        sc = (np.ones(wl.hkv, np.float32), np.ones(wl.hkv, np.float32))
    else:
        r = np.random.default_rng(9)
        sc = (r.uniform(0.004, 0.02, wl.hkv).astype(np.float32),
              r.uniform(0.002, 0.01, wl.hkv).astype(np.float32))
    case = _case(wl, fp8_scales=sc)
    seqs = [0, 5, 17, 31]
    _check_pages(case, seqs)
    if scales == "tight":
        kc, vc = _oracle_codes(case, 0)
        assert ((kc & 0x7F) == 0x7E).mean() > 0.001 and ((vc & 0x7F) == 0x7E).mean() > 0.01
    _check_decode(case, seqs)


@pytest.mark.parametrize("name", ["llama3.1-8b-decode", "qwen2.5-7b-shared-prefix", "llama3-70b"])
def test_fp8_full_size_sampled(name):
    _print_case("fp8_full_size_sampled", workload=name)
    case = _case(W.WORKLOADS[name])
    r = np.random.default_rng(0)
    seqs = {0, len(case.ctx) - 1, int(np.argmin(case.ctx)), int(np.argmax(case.ctx))}
    seqs |= set(int(x) for x in r.choice(len(case.ctx), size=2, replace=False))
    if len(case.plan.sharing):
        seqs.add(int(case.plan.sharing[0]))
    seqs = sorted(seqs)
    _check_pages(case, seqs)
    _check_decode(case, seqs)


def test_fp8_decode_steps_with_append():
    """One token per sequence appended per step (filling pages one slot at a
    time, crossing into new pages), then decoded."""
    _print_case("fp8_decode_steps_with_append")
    base = W.WORKLOADS["llama3.1-8b-decode"]
    wl = W.Workload("f8-8b-steps", 1, 8, base.hq, base.hkv, base.ctx, base.k_outliers, seed=base.seed)
    ctx0 = W.context_lengths(wl)
    steps = 20
    case = LayerCase(wl, ctx_lens=ctx0, extra_tokens=steps, kind="fp8")
    case.cache.pages.fill_(NAN_BYTE)
    case.prefill()
    new = []
    for s in range(steps):
        k, v = W.new_tokens(wl, 0, s, "cuda", case.mult)
        new.append((k.cpu(), v.cpu()))
        cu = torch.arange(wl.batch + 1, dtype=torch.int32, device="cuda")
        sl = torch.tensor((ctx0 + s).astype(np.int32), device="cuda")
        case.cache.append(k.contiguous(), v.contiguous(), cu, sl, 1, case.block_table)
    case.ctx = ctx0 + steps
    case.ctx_gpu = torch.from_numpy(case.ctx.astype(np.int32)).cuda()
    out = case.decode().float().cpu().numpy()
    got, want = [], []
    for b in range(wl.batch):
        k0, v0 = (x.cpu() for x in W.sequence_kv(wl, 0, b, int(ctx0[b]), "cuda", case.mult))
        k = torch.cat([k0] + [x[0][b:b + 1] for x in new]).numpy()
        v = torch.cat([v0] + [x[1][b:b + 1] for x in new]).numpy()
        kc, vc = ofp8.fp8_sequence(k, v, case.k_scale, case.v_scale)
        gk, gv = layout.read_fp8_chunks(case.gpu_fp8_pages(b))
        n = int(case.ctx[b])
        for p in range(int(ctx0[b]) // 16, gk.shape[0]):                 # pages the steps wrote
            t0, t1 = 16 * p, min(n, 16 * p + 16)
            assert np.array_equal(gk[p, :, :t1 - t0], kc[t0:t1].transpose(1, 0, 2))
            assert np.array_equal(gv[p, :, :t1 - t0], vc[t0:t1].transpose(1, 0, 2))
        kh, vh = ofp8.fp8_dequantized(kc, vc, case.k_scale, case.v_scale)
        got.append(out[b])
        want.append(oracle.decode_attention(case.q[b].cpu().numpy(), kh, vh))
    ok, max_abs, rel = parity.attention_ok(np.stack(got), np.stack(want))
    assert ok, (max_abs, rel)
