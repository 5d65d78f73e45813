"""2-bit KIVI pages vs the oracle (bits=2), through the C ABI (libs4kv.so).

The int4 cases with 2-bit codes: codes, fp16 scales/zeros and tails bit-exact
(read back through the 2-bit page format of include/s4kv.h); attention within
the decode bar (2e-3 max-abs, 1e-3 relative L2) over the oracle's dequantized
2-bit cache. Every group width and layout path (G up to 4, up to 8, above 8),
bulk prefill and ragged appends, the full-size shapes on sampled sequences.
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
    case = LayerCase(wl, kind="kivi2", **kw)
    case.prefill()
    return case


def _check_pages(case, seqs):
    for b in seqs:
        want = case.oracle_seq(b)
        bad = parity.page_mismatches(case.gpu_chunks(b), want["pages"], bits=2)
        assert not bad, f"seq {b}: page fields differ: {bad}"
        pad = case.gpu_chunks(b)[..., 1600:]
        assert not pad.any(), f"seq {b}: padding not zero"
        tk, tv = case.gpu_tail(b)
        assert np.array_equal(tk.view(np.uint16), want["tail_k"].view(np.uint16)), f"seq {b}: tail K"
        assert np.array_equal(tv.view(np.uint16), want["tail_v"].view(np.uint16)), f"seq {b}: tail V"


def _check_decode(case, seqs):
    out = case.decode().float().cpu().numpy()
    got = np.concatenate([out[b] for b in seqs])
    want = np.concatenate([case.oracle_out(b) for b in seqs])
    assert np.isfinite(got).all(), "non-finite output"
    ok, max_abs, rel = parity.attention_ok(got, want)
    print(f"  kivi2 decode max_abs={max_abs:.2e} rel_l2={rel:.2e} outputs={len(got)}", flush=True)
    assert ok, f"attention out of tolerance: max_abs={max_abs:.3e} rel_l2={rel:.3e}"


@pytest.mark.parametrize("name", ["tiny", "llama3.2-3b-layer"])
def test_kivi2_pages_and_decode(name):
    _print_case("kivi2_pages_and_decode", workload=name)
    case = _case(W.WORKLOADS[name])
    _check_pages(case, range(case.wl.batch))
    _check_decode(case, range(case.wl.batch))


@pytest.mark.parametrize("g", [1, 3, 4, 7, 8, 16])
def test_kivi2_edge_contexts(g):
    _print_case("kivi2_edge_contexts", group=g)
    ctx = np.array([1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257, 1000, 4111], dtype=np.int64)
    hkv = 2
    wl = W.Workload(f"k2-edge-g{g}", 1, len(ctx), g * hkv, hkv, ("fixed", 1),
                    ("frac", 0.02, 8.0, 20.0), seed=90 + g)
    case = _case(wl, ctx_lens=ctx)
    _check_pages(case, range(wl.batch))
    _check_decode(case, range(wl.batch))


def test_kivi2_append_chunks_match_bulk():
    """Ragged appends give the bulk prefill's pages and tails, bit for bit."""
    _print_case("kivi2_append_chunks")
    ctx = np.array([1, 15, 16, 17, 40, 77, 130], dtype=np.int64)
    wl = W.Workload("k2-ragged", 1, len(ctx), 8, 2, ("fixed", 1), ("frac", 0.02, 8.0, 20.0), seed=12)
    bulk = _case(wl, ctx_lens=ctx)
    inc = LayerCase(wl, ctx_lens=ctx, kind="kivi2")
    seqs_kv = [inc.seq_kv(b) for b in range(wl.batch)]
    r = np.random.default_rng(6)
    pos = np.zeros(wl.batch, dtype=np.int64)
    while (pos < ctx).any():
        n = np.minimum(r.integers(0, 23, size=wl.batch), ctx - pos)
        ks = [seqs_kv[b][0][pos[b]:pos[b] + n[b]] for b in range(wl.batch)]
        vs = [seqs_kv[b][1][pos[b]:pos[b] + n[b]] for b in range(wl.batch)]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(n)]).astype(np.int32), device="cuda")
        sl = torch.tensor(pos.astype(np.int32), device="cuda")
        if n.sum() > 0:
            inc.cache.append(torch.cat(ks).contiguous(), torch.cat(vs).contiguous(), cu, sl,
                             int(n.max()), inc.block_table)
        pos += n
    torch.cuda.synchronize()
    for b in range(wl.batch):
        assert np.array_equal(bulk.gpu_chunks(b), inc.gpu_chunks(b)), f"seq {b}: pages differ"
        for x, y in zip(bulk.gpu_tail(b), inc.gpu_tail(b)):
            assert np.array_equal(x.view(np.uint16), y.view(np.uint16)), f"seq {b}: tails differ"
    _check_pages(inc, range(wl.batch))
    _check_decode(inc, range(wl.batch))


@pytest.mark.parametrize("name", ["llama3.1-8b-decode", "qwen2.5-7b-shared-prefix", "llama3-70b"])
def test_kivi2_full_size_sampled(name):
    _print_case("kivi2_full_size_sampled", workload=name)
    case = _case(W.WORKLOADS[name])
    r = np.random.default_rng(0)
    seqs = {0, len(case.ctx) - 1, int(np.argmin(case.ctx)), int(np.argmax(case.ctx))}
    seqs |= set(int(x) for x in r.choice(len(case.ctx), size=2, replace=False))
    if len(case.plan.sharing):
        seqs.add(int(case.plan.sharing[0]))
    seqs = sorted(seqs)
    _check_pages(case, seqs)
    _check_decode(case, seqs)


def test_kivi2_and_int4_share_tails_and_decode_shape():
    """The two code widths of the same tokens: identical fp16 tails, and the
    2-bit decode stays within the 2-bit oracle's bar while differing from the
    int4 result by the coarser codes."""
    _print_case("kivi2_vs_int4")
    wl = W.WORKLOADS["llama3.2-3b-layer"]
    a = LayerCase(wl)
    a.prefill()
    k2 = _case(wl)
    for b in (0, 7):
        for x, y in zip(a.gpu_tail(b), k2.gpu_tail(b)):
            assert np.array_equal(x.view(np.uint16), y.view(np.uint16))
    oa = a.decode().float().cpu().numpy()
    ob = k2.decode().float().cpu().numpy()
    assert np.abs(oa - ob).max() > 1e-3           # the codes really are coarser
