"""Multi-query attention over the int4 cache vs the oracle, through the C ABI.

T_b new tokens per sequence, already appended (the last T_b cache positions),
attend causally over the dequantized pages and the fp16 tail. The reference is
the oracle's multiquery_attention over the oracle's dequantized cache; the bar
is the decode bar (2e-3 max-abs, 1e-3 relative L2). Ragged token counts,
causal limits inside full pages, across page boundaries and inside the tail,
and every column count up to 16 are covered; so are token counts that need
more than 16 matrix-core columns per KV head (streamed as column tiles), up
to whole causal prefill chunks.
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


def _queries(wl, t_counts, seed):
    total = int(np.sum(t_counts))
    q = W.normal_fp16((total, wl.hq, wl.head_dim), seed, "cuda")
    cu = np.concatenate([[0], np.cumsum(t_counts)]).astype(np.int32)
    return q, cu


def _run(case, t_counts, max_q, seed):
    q, cu = _queries(case.wl, t_counts, seed)
    cu_g = torch.from_numpy(cu).cuda()
    out = case.cache.attend(q, cu_g, max_q, case.block_table, case.ctx_gpu, int(case.ctx.max()))
    torch.cuda.synchronize()
    return q.cpu().numpy(), cu, out.float().cpu().numpy()


def _check(case, seqs, q, cu, out):
    got, want = [], []
    for b in seqs:
        kh, vh = oracle.dequantized_sequence(case.oracle_seq(b))
        rows = slice(cu[b], cu[b + 1])
        want.append(oracle.multiquery_attention(q[rows], kh, vh).reshape(-1, case.wl.head_dim))
        got.append(out[rows].reshape(-1, case.wl.head_dim))
    got, want = np.concatenate(got), np.concatenate(want)
    assert np.isfinite(got).all(), "non-finite output"
    ok, max_abs, rel = parity.attention_ok(got, want)
    print(f"  mq max_abs={max_abs:.2e} rel_l2={rel:.2e} outputs={len(got)}", flush=True)
    assert ok, f"attention out of tolerance: max_abs={max_abs:.3e} rel_l2={rel:.3e}"


@pytest.mark.parametrize("t", [1, 2, 3, 4])
def test_mq_tiny(t):
    _print_case("mq_tiny", t=t)
    case = LayerCase(W.WORKLOADS["tiny"])
    case.prefill()
    q, cu, out = _run(case, [t], t, seed=500 + t)
    _check(case, [0], q, cu, out)


@pytest.mark.parametrize("g,max_q", [(1, 16), (1, 5), (2, 8), (3, 5), (4, 4), (5, 3), (8, 2),
                                     (16, 1)])
def test_mq_edge_contexts(g, max_q):
    """Causal limits in full pages, at page edges and in the tail, with ragged
    token counts 1 .. max_q."""
    _print_case("mq_edge_contexts", group=g, max_q=max_q)
    ctx = np.array([16, 17, 31, 32, 33, 47, 255, 256, 257, 1000, 4111, 18, 100], dtype=np.int64)
    hkv = 2
    wl = W.Workload(f"mq-edge-g{g}", 1, len(ctx), g * hkv, hkv, ("fixed", 1),
                    ("frac", 0.02, 8.0, 20.0), seed=80 + g)
    case = LayerCase(wl, ctx_lens=ctx)
    case.prefill()
    t_counts = np.array([1 + (b % max_q) for b in range(len(ctx))])
    t_counts = np.minimum(t_counts, ctx)
    t_counts[0] = max_q                       # one sequence uses every column
    q, cu, out = _run(case, t_counts, max_q, seed=600 + g)
    _check(case, range(len(ctx)), q, cu, out)


def test_mq_one_token_matches_decode():
    """With one new token per sequence the step is the decode step."""
    _print_case("mq_one_token_matches_decode")
    case = LayerCase(W.WORKLOADS["llama3.2-3b-layer"])
    case.prefill()
    dec = case.decode().float().cpu().numpy()
    q, cu = case.q, np.arange(case.wl.batch + 1, dtype=np.int32)
    out = case.cache.attend(q.reshape(-1, case.wl.hq, case.wl.head_dim).contiguous(),
                            torch.from_numpy(cu).cuda(), 1, case.block_table, case.ctx_gpu,
                            int(case.ctx.max()))
    torch.cuda.synchronize()
    diff = float(np.abs(out.float().cpu().numpy() - dec).max())
    print(f"  mq(T=1) vs decode max |diff| = {diff:.2e}", flush=True)
    assert diff <= 1e-3


@pytest.mark.parametrize("name,max_q", [("llama3.1-8b-decode", 4), ("qwen2.5-7b-shared-prefix", 2),
                                        ("llama3-70b", 2)])
def test_mq_full_size_sampled(name, max_q):
    """Speculative-verify shapes: max_q new tokens per sequence (ragged), full
    workload size, sampled sequences checked."""
    _print_case("mq_full_size_sampled", workload=name, max_q=max_q)
    case = LayerCase(W.WORKLOADS[name])
    case.prefill()
    r = np.random.default_rng(1)
    t_counts = r.integers(1, max_q + 1, size=case.wl.batch)
    t_counts[0] = max_q
    q, cu, out = _run(case, t_counts, max_q, seed=700)
    seqs = {0, len(case.ctx) - 1, int(np.argmin(case.ctx)), int(np.argmax(case.ctx))}
    seqs |= set(int(x) for x in r.choice(len(case.ctx), size=2, replace=False))
    if len(case.plan.sharing):
        seqs.add(int(case.plan.sharing[0]))
    _check(case, sorted(seqs), q, cu, out)


@pytest.mark.parametrize("g,max_q", [(1, 40), (3, 64), (4, 64), (8, 33), (16, 9)])
def test_mq_wide_tiles(g, max_q):
    """More tokens per sequence than 16 / G: the columns go out in tiles of
    whole tokens (16 / G per tile), each tile streaming only the pages up to
    its last token. Ragged counts (a tile may be partly or wholly unused),
    contexts where early tiles stop inside a full page, at a page edge or in
    the tail."""
    _print_case("mq_wide_tiles", group=g, max_q=max_q)
    ctx = np.array([max_q, max_q + 1, 100, 257, 1000, 2000, 64, 47], dtype=np.int64)
    hkv = 2
    wl = W.Workload(f"mq-wide-g{g}", 1, len(ctx), g * hkv, hkv, ("fixed", 1),
                    ("frac", 0.02, 8.0, 20.0), seed=90 + g)
    case = LayerCase(wl, ctx_lens=ctx)
    case.prefill()
    r = np.random.default_rng(g)
    t_counts = np.minimum(r.integers(1, max_q + 1, size=len(ctx)), ctx)
    t_counts[0] = max_q                      # the whole context is new: a first prefill chunk
    t_counts[1] = max_q
    t_counts[4] = 1
    q, cu, out = _run(case, t_counts, max_q, seed=800 + g)
    _check(case, range(len(ctx)), q, cu, out)


def test_mq_prefill_chunks_cover_a_sequence():
    """Chunked prefill: a 700-token sequence appended and attended in chunks of
    256, 256 and 188 tokens gives, token for token, the causal attention of the
    whole sequence (each chunk against everything before it)."""
    _print_case("mq_prefill_chunks")
    wl = W.Workload("mq-chunks", 1, 1, 32, 8, ("fixed", 1), ("frac", 0.02, 8.0, 20.0), seed=97)
    full = LayerCase(wl, ctx_lens=[700])
    k_all, v_all = full.seq_kv(0)
    q_all = W.normal_fp16((700, wl.hq, wl.head_dim), 4343, "cuda")
    pos, outs = 0, []
    for n in (256, 256, 188):
        cu_new = torch.tensor([0, n], dtype=torch.int32, device="cuda")
        slot = torch.tensor([pos], dtype=torch.int32, device="cuda")
        full.cache.append(k_all[pos:pos + n].contiguous(), v_all[pos:pos + n].contiguous(), cu_new,
                          slot, n, full.block_table)
        ctx = torch.tensor([pos + n], dtype=torch.int32, device="cuda")
        outs.append(full.cache.attend(q_all[pos:pos + n].contiguous(), cu_new, n, full.block_table,
                                      ctx, pos + n))
        pos += n
    torch.cuda.synchronize()
    got = torch.cat(outs).float().cpu().numpy()
    kh, vh = oracle.dequantized_sequence(oracle.sequence_cache(k_all.cpu().numpy(),
                                                               v_all.cpu().numpy()))
    want = oracle.multiquery_attention(q_all.cpu().numpy(), kh, vh)
    ok, max_abs, rel = parity.attention_ok(got.reshape(-1, 128), want.reshape(-1, 128))
    print(f"  chunked prefill max_abs={max_abs:.2e} rel_l2={rel:.2e}", flush=True)
    assert ok, (max_abs, rel)


@pytest.mark.timeout(600)
def test_mq_wide_full_size_sampled():
    """The 8B-shaped layer with 128 new tokens per sequence (32 tiles of 4
    tokens per sequence, 4096 virtual sequences); two sequences checked."""
    _print_case("mq_wide_full_size_sampled", workload="llama3.1-8b-decode", max_q=128)
    case = LayerCase(W.WORKLOADS["llama3.1-8b-decode"])
    case.prefill()
    t_counts = np.full(case.wl.batch, 128)
    t_counts[5] = 77
    q, cu, out = _run(case, t_counts, 128, seed=900)
    _check(case, [0, 5], q, cu, out)
