"""The read probe (a measurement aid of libs4kv.so) runs through the C ABI and
skips chunk ids outside its pool instead of reading past it."""

import pytest
import torch

from int4_kivi_quantized_amd import s4kv

pytestmark = pytest.mark.gpu


def test_probe_read_runs_and_skips_out_of_range_ids():
    print("[case] probe_read", flush=True)
    pool = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")       # 256 chunks
    ids = torch.arange(256, dtype=torch.int32, device="cuda")
    ids[5], ids[77], ids[200] = -1, 256, 2**31 - 1                       # skipped by the kernel
    for nt in (True, False):
        s4kv.s4kv_probe_read(pool, ids, 64, 4, nt)
    torch.cuda.synchronize()
    assert int(pool.sum()) == 0                                         # read only
