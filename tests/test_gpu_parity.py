"""GPU path vs CPU oracle, through the C ABI (libs4kv.so).

Quantization (bulk prefill and append): codes, fp16 scales/zeros and tails
bit-exact. Decode: attention within 2e-3 max-abs and 1e-3 relative L2.
Small workloads are checked in full; the full-size workloads on sampled
sequences, with the same launch configuration the benchmark uses.
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


def _check_pages(case, seqs):
    for b in seqs:
        want = case.oracle_seq(b)
        bad = parity.page_mismatches(case.gpu_chunks(b), want["pages"])
        assert not bad, f"seq {b}: page fields differ: {bad}"
        tk, tv = case.gpu_tail(b)
        assert np.array_equal(tk.view(np.uint16), want["tail_k"].view(np.uint16)), f"seq {b}: tail K"
        assert np.array_equal(tv.view(np.uint16), want["tail_v"].view(np.uint16)), f"seq {b}: tail V"


def _sampled(case, n_rand=2, seed=0):
    ctx = case.ctx
    r = np.random.default_rng(seed)
    pick = {0, len(ctx) - 1, int(np.argmin(ctx)), int(np.argmax(ctx))}
    pick |= set(int(x) for x in r.choice(len(ctx), size=min(n_rand, len(ctx)), replace=False))
    return sorted(pick)


def _check_decode(case, seqs, heads=None):
    out = case.decode().float().cpu().numpy()
    got, want = [], []
    for b in seqs:
        ref = case.oracle_out(b, heads)
        hs = range(case.wl.hq) if heads is None else heads
        for j in hs:
            got.append(out[b, j])
            want.append(ref[j])
    ok, max_abs, rel = parity.attention_ok(np.stack(got), np.stack(want))
    print(f"  decode max_abs={max_abs:.2e} rel_l2={rel:.2e} outputs={len(got)}", flush=True)
    assert ok, f"attention out of tolerance: max_abs={max_abs:.3e} rel_l2={rel:.3e}"


# --------------------------------------------------------------- small, in full

@pytest.mark.parametrize("name", ["tiny", "llama3.2-3b-layer"])
def test_prefill_pages_bitexact(name):
    _print_case("prefill_bitexact", workload=name)
    case = LayerCase(W.WORKLOADS[name])
    case.prefill()
    _check_pages(case, range(case.wl.batch))


@pytest.mark.parametrize("name", ["tiny", "llama3.2-3b-layer"])
def test_decode_parity(name):
    _print_case("decode_parity", workload=name)
    case = LayerCase(W.WORKLOADS[name])
    case.prefill()
    _check_decode(case, range(case.wl.batch))


# --------------------------------------------------------------- full size, sampled

def _check_layer_full(case):
    """Every page and tail of every sequence bit-exact, and the output of every
    sequence and query head within the attention bar; the oracle runs per
    sequence on a thread pool (numpy releases the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    wl = case.wl
    out = case.decode().float().cpu().numpy()
    kvs = [tuple(x.cpu().numpy() for x in case.seq_kv(b)) for b in range(wl.batch)]
    chunks = [case.gpu_chunks(b) for b in range(wl.batch)]
    tails = [case.gpu_tail(b) for b in range(wl.batch)]
    q = case.q.cpu().numpy()

    def one(b):
        c = oracle.sequence_cache(*kvs[b])
        bad = parity.page_mismatches(chunks[b], c["pages"])
        tk, tv = tails[b]
        tail_ok = (np.array_equal(tk.view(np.uint16), c["tail_k"].view(np.uint16))
                   and np.array_equal(tv.view(np.uint16), c["tail_v"].view(np.uint16)))
        kh, vh = oracle.dequantized_sequence(c)
        return bad, tail_ok, oracle.decode_attention(q[b], kh, vh)

    with ThreadPoolExecutor(8) as ex:
        res = list(ex.map(one, range(wl.batch)))
    for b, (bad, tail_ok, _) in enumerate(res):
        assert not bad, f"seq {b}: page fields differ: {bad}"
        assert tail_ok, f"seq {b}: tail differs"
    ok, max_abs, rel = parity.attention_ok(out, np.stack([r[2] for r in res]))
    print(f"  {wl.batch} sequences x {wl.hq} heads: pages and tails bit-exact, "
          f"decode max_abs={max_abs:.2e} rel_l2={rel:.2e}", flush=True)
    assert ok, f"attention out of tolerance: max_abs={max_abs:.3e} rel_l2={rel:.3e}"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,layer", [("llama3-70b", 0), ("llama3-70b", 79),
                                        ("qwen2.5-7b-shared-prefix", 0)])
def test_full_layer(name, layer):
    """Whole layers: the first and last layer of the 70B-shaped workload (B16,
    32K contexts, G = 8) and the shared-prefix layer (G = 7; aliased prefix
    pages are read by every sharing sequence)."""
    _print_case("full_layer", workload=name, layer=layer)
    case = LayerCase(W.WORKLOADS[name], layer=layer)
    case.prefill()
    if len(case.plan.sharing):
        b = int(case.plan.sharing[0])
        assert set(case.plan.block_table[b, :4]) <= set(case.plan.prefix_pages.tolist())
    _check_layer_full(case)


@pytest.mark.parametrize("name", ["llama3.1-8b-decode"])
def test_full_size_sampled(name):
    _print_case("full_size_sampled", workload=name)
    case = LayerCase(W.WORKLOADS[name])
    case.prefill()
    seqs = _sampled(case)
    _check_pages(case, seqs)
    if len(case.plan.sharing):
        # aliased pages: a sharing sequence reads the prefix's physical pages
        b = int(case.plan.sharing[0])
        assert set(case.plan.block_table[b, :4]) <= set(case.plan.prefix_pages.tolist())
        seqs = sorted(set(seqs) | {b})
    _check_decode(case, seqs)


# --------------------------------------------------------------- append path

def _small_wl(name, batch, hq, hkv, seed=11):
    return W.Workload(name, 1, batch, hq, hkv, ("fixed", 1), ("frac", 0.02, 8.0, 20.0), seed=seed)


def test_append_chunks_match_bulk_and_oracle():
    """Tokens arriving in ragged chunks (first page partial, full middle pages,
    partial last page) give the same pages and tails as one bulk prefill."""
    _print_case("append_chunks")
    ctx = np.array([1, 15, 16, 17, 40, 77, 130], dtype=np.int64)
    wl = _small_wl("ragged", len(ctx), 8, 2)
    bulk = LayerCase(wl, ctx_lens=ctx)
    bulk.prefill()
    inc = LayerCase(wl, ctx_lens=ctx)
    seqs_kv = [inc.seq_kv(b) for b in range(wl.batch)]
    r = np.random.default_rng(5)
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


def test_decode_steps_with_append():
    """Decode steps of the 8B-shaped workload at reduced batch: one token per
    sequence is appended each step (crossing page flushes), then decoded."""
    _print_case("decode_steps_with_append")
    base = W.WORKLOADS["llama3.1-8b-decode"]
    wl = W.Workload("8b-steps", 1, 8, base.hq, base.hkv, base.ctx, base.k_outliers, seed=base.seed)
    ctx0 = W.context_lengths(wl)
    steps = 20
    case = LayerCase(wl, ctx_lens=ctx0, extra_tokens=steps)
    case.prefill()
    new = []
    for s in range(steps):
        k, v = W.new_tokens(wl, 0, s, "cuda", case.mult)
        new.append((k, v))
        cu = torch.arange(wl.batch + 1, dtype=torch.int32, device="cuda")
        sl = torch.tensor((ctx0 + s).astype(np.int32), device="cuda")
        case.cache.append(k.contiguous(), v.contiguous(), cu, sl, 1, case.block_table)
    case.ctx = ctx0 + steps
    case.ctx_gpu = torch.from_numpy(case.ctx.astype(np.int32)).cuda()
    out = case.decode().float().cpu().numpy()
    got, want = [], []
    for b in range(wl.batch):
        k0, v0 = W.sequence_kv(wl, 0, b, int(ctx0[b]), "cuda", case.mult)
        k = torch.cat([k0] + [x[0][b:b + 1] for x in new]).cpu().numpy()
        v = torch.cat([v0] + [x[1][b:b + 1] for x in new]).cpu().numpy()
        c = oracle.sequence_cache(k, v)
        bad = parity.page_mismatches(case.gpu_chunks(b), c["pages"])
        assert not bad, f"seq {b}: {bad}"
        kh, vh = oracle.dequantized_sequence(c)
        ref = oracle.decode_attention(case.q[b].cpu().numpy(), kh, vh)
        got.append(out[b])
        want.append(ref)
    ok, max_abs, rel = parity.attention_ok(np.stack(got), np.stack(want))
    assert ok, (max_abs, rel)


# --------------------------------------------------------------- edge cases, invariants

@pytest.mark.parametrize("g", [1, 3, 4, 7, 8, 16])
def test_decode_edge_contexts(g):
    _print_case("edge_contexts", group=g)
    ctx = np.array([1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257, 1000, 4111], dtype=np.int64)
    hkv = 2
    wl = _small_wl(f"edge-g{g}", len(ctx), g * hkv, hkv, seed=20 + g)
    case = LayerCase(wl, ctx_lens=ctx)
    case.prefill()
    _check_pages(case, range(wl.batch))
    _check_decode(case, range(wl.batch))


def test_decode_invariants():
    _print_case("invariants")
    ctx = np.array([700, 1601, 33, 2048], dtype=np.int64)
    wl = _small_wl("inv", len(ctx), 16, 2, seed=40)
    a = LayerCase(wl, ctx_lens=ctx)
    a.prefill()
    oa = a.decode()
    # max_ctx only bounds the launch; a larger bound must not move the result
    ob = a.decode(max_ctx=16 * a.plan.max_pages)
    assert torch.allclose(oa.float(), ob.float(), atol=2e-3, rtol=0)
    # same pages behind a different permutation of the pool: identical output
    import dataclasses
    wl2 = dataclasses.replace(wl, seed=41)
    b = LayerCase(wl2, ctx_lens=ctx)
    b.mult = a.mult
    b.q = a.q
    b.seq_kv = a.seq_kv
    assert not np.array_equal(a.plan.block_table, b.plan.block_table)
    b.prefill()
    assert torch.equal(oa, b.decode()), "pool permutation changed the output"
    # query heads with identical q give identical outputs
    a.q[:, 1] = a.q[:, 0]
    oc = a.decode()
    assert torch.equal(oc[:, 0], oc[:, 1])
