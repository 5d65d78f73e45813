"""fp16 control path vs the oracle, through the C ABI (libs4kv.so).

Append: every defined token slot of the fp16 pool holds the input bits (K
rows, V transposed). The pool is filled with NaN first, so a slot the kernels
wrongly read, or an undefined slot of a partial page that reached the
arithmetic, shows up in the outputs. Decode: attention over the fp16 values
within 2e-3 max-abs and 1e-3 relative L2 of the oracle (plain softmax
attention in float64 over the same fp16 K and V).
"""

import numpy as np
import pytest
import torch

import oracle
import workload as W
from tests import parity
from tests.gpu_harness import LayerCase

pytestmark = pytest.mark.gpu


def _print_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _case(wl, **kw):
    case = LayerCase(wl, kind="fp16", **kw)
    case.cache.pages.fill_(float("nan"))
    case.prefill()
    return case


def _check_pages(case, seqs):
    for b in seqs:
        k, v = case.seq_kv(b)
        k = k.cpu().numpy().view(np.uint16)
        v = v.cpu().numpy().view(np.uint16)
        got = case.gpu_fp16_pages(b).view(np.uint16)      # [pages, Hkv, 4096]
        n = int(case.ctx[b])
        for p in range(got.shape[0]):
            t0, t1 = 16 * p, min(n, 16 * p + 16)
            kb = got[p, :, :2048].reshape(-1, 16, 128)     # [Hkv, token, channel]
            vb = got[p, :, 2048:].reshape(-1, 128, 16)     # [Hkv, channel, token]
            want_k = k[t0:t1].transpose(1, 0, 2)           # [Hkv, tokens, 128]
            want_v = v[t0:t1].transpose(1, 2, 0)           # [Hkv, 128, tokens]
            assert np.array_equal(kb[:, :t1 - t0], want_k), f"seq {b} page {p}: K slots differ"
            assert np.array_equal(vb[:, :, :t1 - t0], want_v), f"seq {b} page {p}: V slots differ"


def _check_decode(case, seqs):
    out = case.decode().float().cpu().numpy()
    got, want = [], []
    for b in seqs:
        k, v = case.seq_kv(b)
        ref = oracle.decode_attention(case.q[b].cpu().numpy(), k.cpu().numpy().astype(np.float32),
                                      v.cpu().numpy().astype(np.float32))
        got.append(out[b])
        want.append(ref)
    got, want = np.concatenate(got), np.concatenate(want)
    assert np.isfinite(got).all(), "non-finite output"
    ok, max_abs, rel = parity.attention_ok(got, want)
    print(f"  fp16 decode max_abs={max_abs:.2e} rel_l2={rel:.2e} outputs={len(got)}", flush=True)
    assert ok, f"attention out of tolerance: max_abs={max_abs:.3e} rel_l2={rel:.3e}"


@pytest.mark.parametrize("name", ["tiny", "llama3.2-3b-layer"])
def test_fp16_pages_and_decode(name):
    _print_case("fp16_pages_and_decode", workload=name)
    case = _case(W.WORKLOADS[name])
    _check_pages(case, range(case.wl.batch))
    _check_decode(case, range(case.wl.batch))


@pytest.mark.parametrize("g", [1, 3, 4, 7, 8, 16])
def test_fp16_edge_contexts(g):
    _print_case("fp16_edge_contexts", group=g)
    ctx = np.array([1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257, 1000, 4111], dtype=np.int64)
    hkv = 2
    wl = W.Workload(f"f16-edge-g{g}", 1, len(ctx), g * hkv, hkv, ("fixed", 1),
                    ("frac", 0.02, 8.0, 20.0), seed=60 + g)
    case = _case(wl, ctx_lens=ctx)
    _check_pages(case, range(wl.batch))
    _check_decode(case, range(wl.batch))


@pytest.mark.parametrize("name", ["llama3.1-8b-decode", "qwen2.5-7b-shared-prefix", "llama3-70b"])
def test_fp16_full_size_sampled(name):
    _print_case("fp16_full_size_sampled", workload=name)
    case = _case(W.WORKLOADS[name])
    r = np.random.default_rng(0)
    seqs = {0, len(case.ctx) - 1, int(np.argmin(case.ctx)), int(np.argmax(case.ctx))}
    seqs |= set(int(x) for x in r.choice(len(case.ctx), size=2, replace=False))
    if len(case.plan.sharing):
        seqs.add(int(case.plan.sharing[0]))
    seqs = sorted(seqs)
    _check_pages(case, seqs)
    _check_decode(case, seqs)


def test_fp16_decode_steps_with_append():
    """One token per sequence appended per step (filling pages one slot at a
    time, crossing into new pages), then decoded."""
    _print_case("fp16_decode_steps_with_append")
    base = W.WORKLOADS["llama3.1-8b-decode"]
    wl = W.Workload("f16-8b-steps", 1, 8, base.hq, base.hkv, base.ctx, base.k_outliers, seed=base.seed)
    ctx0 = W.context_lengths(wl)
    steps = 20
    case = LayerCase(wl, ctx_lens=ctx0, extra_tokens=steps, kind="fp16")
    case.cache.pages.fill_(float("nan"))
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
        got.append(out[b])
        want.append(oracle.decode_attention(case.q[b].cpu().numpy(), k.astype(np.float32),
                                            v.astype(np.float32)))
    ok, max_abs, rel = parity.attention_ok(np.stack(got), np.stack(want))
    assert ok, (max_abs, rel)
