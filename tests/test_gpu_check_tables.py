"""s4kv_check_tables: the on-device check of the block table and context
lengths that the append and decode kernels trust (include/s4kv.h, "Table
checks"). Valid tables report no fault; planted and random faults are counted
exactly as a plain host loop over the same definition counts them, with the
same first faulty (sequence, page). Every table entry the kernel reads lies
inside the table, whatever it holds."""

import numpy as np
import pytest
import torch

import workload as W
from int4_kivi_quantized_amd import Shape, s4kv

pytestmark = pytest.mark.gpu

PAGE = 16


def host_report(block_table, ctx, num_pages, max_pages, max_ctx):
    """Fault counts and first fault, by the definition in s4kv.h, one entry at a time."""
    bad_len = bad_ids = 0
    first = None
    limit = max_pages * PAGE
    for b in range(len(ctx)):
        c = int(ctx[b])
        faults = []
        if c < 0 or c > limit or (max_ctx > 0 and c > max_ctx):
            bad_len += 1
            faults.append(-1)
        used = (min(max(c, 0), limit) + PAGE - 1) // PAGE
        for p in range(used):
            i = int(block_table[b, p])
            if i < 0 or i >= num_pages:
                bad_ids += 1
                faults.append(p)
        if faults and first is None:
            first = (b, min(faults))
    return [bad_len, bad_ids, -1 if first is None else first[0], -1 if first is None else first[1]]


def run(block_table, ctx, num_pages, max_ctx, hq=24, hkv=8):
    B, max_pages = block_table.shape
    shape = Shape(B, hq, hkv, num_pages, max_pages)
    bt = torch.from_numpy(np.ascontiguousarray(block_table, dtype=np.int32)).cuda()
    cl = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).cuda()
    report = torch.full((4,), 12345, dtype=torch.int32, device="cuda")   # junk: every field is written
    s4kv.s4kv_check_tables(shape, bt, cl, max_ctx, report)
    torch.cuda.synchronize()
    return report.cpu().tolist()


def test_valid_tables_report_no_fault():
    print("[case] check_tables valid", flush=True)
    for name in ("llama3.2-3b-layer", "qwen2.5-7b-shared-prefix", "tiny"):
        wl = W.WORKLOADS[name]
        ctx = W.context_lengths(wl)
        plan = W.plan_pages(wl, ctx, 8)
        got = run(plan.block_table, ctx, plan.num_pages, int(ctx.max()), wl.hq, wl.hkv)
        assert got == [0, 0, -1, -1], (name, got)
        # unused entries past each sequence's pages may hold anything
        bt = plan.block_table.copy()
        for b in range(len(ctx)):
            bt[b, (int(ctx[b]) + PAGE - 1) // PAGE:] = -7
        assert run(bt, ctx, plan.num_pages, 0, wl.hq, wl.hkv) == [0, 0, -1, -1], name


def test_planted_faults_are_counted_and_located():
    print("[case] check_tables planted", flush=True)
    wl = W.WORKLOADS["llama3.2-3b-layer"]
    ctx = W.context_lengths(wl).copy()
    plan = W.plan_pages(wl, ctx, 0)
    bt = plan.block_table.copy()
    n, mp = plan.num_pages, plan.max_pages
    ctx[9] = -1                              # negative length
    ctx[4] = mp * PAGE + 1                   # longer than the table row
    bt[7, 2] = n                             # one past the pool, in use
    bt[7, 0] = -3                            # negative id, in use: the first fault of sequence 7
    bt[11, (int(ctx[11]) + PAGE - 1) // PAGE] = n + 99   # past the sequence's pages: not a fault
    for max_ctx in (0, int(np.sort(ctx)[-3])):
        want = host_report(bt, ctx, n, mp, max_ctx)
        got = run(bt, ctx, n, max_ctx, wl.hq, wl.hkv)
        assert got == want, (max_ctx, got, want)
    assert run(bt, ctx, n, 0, wl.hq, wl.hkv)[2:] == [4, -1]


@pytest.mark.parametrize("seed", range(6))
def test_random_tables_match_host_count(seed):
    print(f"[case] check_tables random seed={seed}", flush=True)
    r = np.random.default_rng(seed)
    B = int(r.integers(1, 1500))
    mp = int(r.integers(1, 600))
    n = int(r.integers(1, 5000))
    ctx = r.integers(-20, mp * PAGE + 40, size=B)
    ok = r.random(B) < 0.7
    ctx[ok] = np.minimum(np.abs(ctx[ok]), mp * PAGE)
    bt = r.integers(0, n, size=(B, mp))
    bad = r.random((B, mp)) < 10.0 / (B * mp) ** 0.5
    bt[bad] = r.choice([-1, -1000, n, n + 1, 2**31 - 1], size=int(bad.sum()))
    max_ctx = int(r.choice([0, int(r.integers(1, mp * PAGE + 1))]))
    want = host_report(bt, ctx, n, mp, max_ctx)
    got = run(bt, ctx, n, max_ctx, 8, 8)
    assert got == want, (B, mp, n, max_ctx, got, want)
