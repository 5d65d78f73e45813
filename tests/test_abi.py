"""The C-ABI library loads, exports every symbol include/s4kv.h declares, and
refuses bad shapes and arguments on the host before any launch (no GPU
needed: none of these calls reaches a kernel)."""

import ctypes
import os
import re

import pytest

from int4_kivi_quantized_amd import s4kv
from int4_kivi_quantized_amd.s4kv import Shape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    inc = os.path.join(ROOT, "include")
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc))
                   if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(s4kv_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_are_exported():
    lib = s4kv.load()
    names = _declared()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/*.h but not exported"
    assert set(names) == set(s4kv.EXPORTED)


def test_library_is_gfx950_only_build():
    path = s4kv.library_path()
    data = open(path, "rb").read()
    assert b"gfx950" in data


GOOD = dict(num_seqs=4, num_q_heads=32, num_kv_heads=8, num_pages=100, max_pages_per_seq=64)


@pytest.mark.parametrize("change,status", [
    ({}, s4kv.S4KV_OK),
    ({"head_dim": 64}, s4kv.S4KV_ERR_UNSUPPORTED),
    ({"head_dim": 256}, s4kv.S4KV_ERR_UNSUPPORTED),
    ({"page_size": 32}, s4kv.S4KV_ERR_UNSUPPORTED),
    ({"num_q_heads": 30}, s4kv.S4KV_ERR_UNSUPPORTED),          # Hq % Hkv != 0
    ({"num_q_heads": 136, "num_kv_heads": 8}, s4kv.S4KV_ERR_UNSUPPORTED),  # G = 17
    ({"num_q_heads": 128, "num_kv_heads": 8}, s4kv.S4KV_OK),   # G = 16
    ({"num_seqs": 0}, s4kv.S4KV_ERR_INVALID_ARG),
    ({"num_pages": 0}, s4kv.S4KV_ERR_INVALID_ARG),
    ({"num_pages": 2**28, "num_kv_heads": 8, "num_q_heads": 32}, s4kv.S4KV_ERR_INVALID_ARG),  # chunk index > int32
    ({"max_pages_per_seq": -1}, s4kv.S4KV_ERR_INVALID_ARG),
    ({"num_kv_heads": 0}, s4kv.S4KV_ERR_INVALID_ARG),
])
def test_validate(change, status):
    args = dict(GOOD)
    args.update(change)
    assert s4kv.s4kv_validate(Shape(**args)) == status


def test_null_shape_and_status_strings():
    lib = s4kv.load()
    assert lib.s4kv_validate(None) == s4kv.S4KV_ERR_INVALID_ARG
    for st in range(5):
        assert len(s4kv.s4kv_status_string(st)) > 0
    assert s4kv.s4kv_status_string(99) == "unknown status"


def test_sizes():
    sh = Shape(**GOOD)
    assert s4kv.s4kv_pool_bytes(sh) == 100 * 8 * 2688
    assert s4kv.s4kv_fp16_pool_bytes(sh) == 100 * 8 * 8192
    assert s4kv.s4kv_fp16_pool_bytes(Shape(**{**GOOD, "page_size": 8})) == 0
    assert s4kv.s4kv_fp8_pool_bytes(sh) == 100 * 8 * 4096
    assert s4kv.s4kv_fp8_pool_bytes(Shape(**{**GOOD, "num_q_heads": 12})) == 0
    assert s4kv.s4kv_tail_bytes(sh) == 4 * 8 * 16 * 128 * 2
    assert s4kv.s4kv_pool_bytes(Shape(**{**GOOD, "head_dim": 64})) == 0
    ws = s4kv.s4kv_decode_workspace_bytes(sh, 1024)
    assert ws >= 4 * 32 * 128 * 4          # at least one split of fp32 partials
    assert s4kv.s4kv_decode_workspace_bytes(sh, 0) == 0
    # a longer context bound never needs less workspace
    assert s4kv.s4kv_decode_workspace_bytes(sh, 1024) >= s4kv.s4kv_decode_workspace_bytes(sh, 16)


def _raw_calls():
    lib = s4kv.load()
    P = ctypes.c_void_p
    fake = P(0x1000)   # never dereferenced: every case below fails host validation
    return lib, P, fake


def test_append_refuses_before_launch():
    lib, P, fake = _raw_calls()
    bad = Shape(**{**GOOD, "head_dim": 96}).c()
    good = Shape(**GOOD).c()
    args = [fake, fake, fake, fake, 1, fake, fake, fake, fake, None]
    assert lib.s4kv_quantize_append(ctypes.byref(bad), *args) == s4kv.S4KV_ERR_UNSUPPORTED
    a = list(args)
    a[0] = None
    assert lib.s4kv_quantize_append(ctypes.byref(good), *a) == s4kv.S4KV_ERR_INVALID_ARG
    a = list(args)
    a[4] = -1
    assert lib.s4kv_quantize_append(ctypes.byref(good), *a) == s4kv.S4KV_ERR_INVALID_ARG
    a = list(args)
    a[4] = 64 * 16 + 1                       # more new tokens than the block table can hold
    assert lib.s4kv_quantize_append(ctypes.byref(good), *a) == s4kv.S4KV_ERR_INVALID_ARG
    a = list(args)
    a[4] = 0                                 # nothing to do: OK without a launch
    assert lib.s4kv_quantize_append(ctypes.byref(good), *a) == s4kv.S4KV_OK


def test_decode_refuses_before_launch():
    lib, P, fake = _raw_calls()
    good = Shape(**GOOD).c()
    ws = s4kv.s4kv_decode_workspace_bytes(Shape(**GOOD), 1000)

    def call(shape=good, max_ctx=1000, ws_bytes=ws, null_at=None):
        ptrs = [fake] * 6
        if null_at is not None:
            ptrs[null_at] = None
        q, pages, tk, tv, bt, cl = ptrs
        return lib.s4kv_paged_decode(ctypes.byref(shape), q, pages, tk, tv, bt, cl, max_ctx,
                                     ctypes.c_float(0.088), fake, fake, ws_bytes, None)

    bad = Shape(**{**GOOD, "num_q_heads": 12}).c()
    assert call(shape=bad) == s4kv.S4KV_ERR_UNSUPPORTED
    assert call(max_ctx=0) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(max_ctx=64 * 16 + 1) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(ws_bytes=ws - 1) == s4kv.S4KV_ERR_WORKSPACE
    for i in range(6):
        assert call(null_at=i) == s4kv.S4KV_ERR_INVALID_ARG


def test_decode_append_refuses_before_launch():
    lib, P, fake = _raw_calls()
    good = Shape(**GOOD).c()
    ws = s4kv.s4kv_decode_workspace_bytes(Shape(**GOOD), 1000)

    def call(shape=good, max_ctx=1000, ws_bytes=ws, null_at=None):
        ptrs = [fake] * 9
        if null_at is not None:
            ptrs[null_at] = None
        q, kn, vn, pages, tk, tv, bt, cl, out = ptrs
        return lib.s4kv_paged_decode_append(ctypes.byref(shape), q, kn, vn, pages, tk, tv, bt, cl,
                                            max_ctx, ctypes.c_float(0.088), out, fake, ws_bytes,
                                            None)

    bad = Shape(**{**GOOD, "num_q_heads": 12}).c()
    assert call(shape=bad) == s4kv.S4KV_ERR_UNSUPPORTED
    assert call(max_ctx=0) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(max_ctx=64 * 16 + 1) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(ws_bytes=ws - 1) == s4kv.S4KV_ERR_WORKSPACE
    for i in range(9):
        assert call(null_at=i) == s4kv.S4KV_ERR_INVALID_ARG


def test_fp16_append_refuses_before_launch():
    lib, P, fake = _raw_calls()
    bad = Shape(**{**GOOD, "num_kv_heads": 5}).c()
    good = Shape(**GOOD).c()
    args = [fake, fake, fake, fake, 1, fake, fake, None]
    assert lib.s4kv_fp16_append(ctypes.byref(bad), *args) == s4kv.S4KV_ERR_UNSUPPORTED
    for i in (0, 1, 2, 3, 5, 6):
        a = list(args)
        a[i] = None
        assert lib.s4kv_fp16_append(ctypes.byref(good), *a) == s4kv.S4KV_ERR_INVALID_ARG
    a = list(args)
    a[4] = 64 * 16 + 1
    assert lib.s4kv_fp16_append(ctypes.byref(good), *a) == s4kv.S4KV_ERR_INVALID_ARG
    a = list(args)
    a[4] = 0
    assert lib.s4kv_fp16_append(ctypes.byref(good), *a) == s4kv.S4KV_OK


def test_fp16_decode_refuses_before_launch():
    lib, P, fake = _raw_calls()
    good = Shape(**GOOD).c()
    ws = s4kv.s4kv_decode_workspace_bytes(Shape(**GOOD), 1000)

    def call(shape=good, max_ctx=1000, ws_bytes=ws, null_at=None):
        ptrs = [fake] * 4
        if null_at is not None:
            ptrs[null_at] = None
        q, pages, bt, cl = ptrs
        return lib.s4kv_fp16_paged_decode(ctypes.byref(shape), q, pages, bt, cl, max_ctx,
                                          ctypes.c_float(0.088), fake, fake, ws_bytes, None)

    bad = Shape(**{**GOOD, "head_dim": 64}).c()
    assert call(shape=bad) == s4kv.S4KV_ERR_UNSUPPORTED
    assert call(max_ctx=0) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(max_ctx=64 * 16 + 1) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(ws_bytes=ws - 1) == s4kv.S4KV_ERR_WORKSPACE
    for i in range(4):
        assert call(null_at=i) == s4kv.S4KV_ERR_INVALID_ARG


def test_fp8_append_refuses_before_launch():
    lib, P, fake = _raw_calls()
    bad = Shape(**{**GOOD, "page_size": 32}).c()
    good = Shape(**GOOD).c()
    # k, v, cu_new, slot, max_new, block_table, k_scale, v_scale, pages, stream
    args = [fake, fake, fake, fake, 1, fake, fake, fake, fake, None]
    assert lib.s4kv_fp8_append(ctypes.byref(bad), *args) == s4kv.S4KV_ERR_UNSUPPORTED
    for i in (0, 1, 2, 3, 5, 6, 7, 8):
        a = list(args)
        a[i] = None
        assert lib.s4kv_fp8_append(ctypes.byref(good), *a) == s4kv.S4KV_ERR_INVALID_ARG
    a = list(args)
    a[4] = -1
    assert lib.s4kv_fp8_append(ctypes.byref(good), *a) == s4kv.S4KV_ERR_INVALID_ARG
    a[4] = 64 * 16 + 1
    assert lib.s4kv_fp8_append(ctypes.byref(good), *a) == s4kv.S4KV_ERR_INVALID_ARG
    a[4] = 0
    assert lib.s4kv_fp8_append(ctypes.byref(good), *a) == s4kv.S4KV_OK


def test_fp8_decode_refuses_before_launch():
    lib, P, fake = _raw_calls()
    good = Shape(**GOOD).c()
    ws = s4kv.s4kv_decode_workspace_bytes(Shape(**GOOD), 1000)

    def call(shape=good, max_ctx=1000, ws_bytes=ws, null_at=None):
        ptrs = [fake] * 8
        if null_at is not None:
            ptrs[null_at] = None
        q, pages, bt, cl, ks, vs, out, wsp = ptrs
        return lib.s4kv_fp8_paged_decode(ctypes.byref(shape), q, pages, bt, cl, max_ctx,
                                         ctypes.c_float(0.088), ks, vs, out, wsp, ws_bytes, None)

    assert call(shape=Shape(**{**GOOD, "num_q_heads": 8 * 17}).c()) == s4kv.S4KV_ERR_UNSUPPORTED
    assert call(max_ctx=0) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(max_ctx=64 * 16 + 1) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(ws_bytes=ws - 1) == s4kv.S4KV_ERR_WORKSPACE
    for i in range(8):
        assert call(null_at=i) == s4kv.S4KV_ERR_INVALID_ARG


def test_probe_refuses_before_launch():
    lib, P, fake = _raw_calls()
    assert lib.s4kv_probe_read(None, 1 << 20, fake, 1, 1, 1, None) == s4kv.S4KV_ERR_INVALID_ARG
    assert lib.s4kv_probe_read(fake, 1 << 20, None, 1, 1, 1, None) == s4kv.S4KV_ERR_INVALID_ARG
    assert lib.s4kv_probe_read(fake, 4095, fake, 1, 1, 1, None) == s4kv.S4KV_ERR_INVALID_ARG
    assert lib.s4kv_probe_read(fake, 1 << 20, fake, 0, 1, 1, None) == s4kv.S4KV_ERR_INVALID_ARG
    assert lib.s4kv_probe_read(fake, 1 << 20, fake, 1, 0, 1, None) == s4kv.S4KV_ERR_INVALID_ARG


def test_kivi2_sizes_and_refusals():
    sh = Shape(**GOOD)
    assert s4kv.s4kv_kivi2_pool_bytes(sh) == 100 * 8 * 1664
    assert s4kv.s4kv_kivi2_pool_bytes(Shape(**{**GOOD, "head_dim": 64})) == 0
    lib, P, fake = _raw_calls()
    good = Shape(**GOOD).c()
    bad = Shape(**{**GOOD, "num_q_heads": 12}).c()
    args = [fake, fake, fake, fake, 1, fake, fake, fake, fake, None]
    assert lib.s4kv_kivi2_quantize_append(ctypes.byref(bad), *args) == s4kv.S4KV_ERR_UNSUPPORTED
    for i in (0, 1, 2, 3, 5, 6, 7, 8):
        a = list(args)
        a[i] = None
        assert lib.s4kv_kivi2_quantize_append(ctypes.byref(good), *a) == s4kv.S4KV_ERR_INVALID_ARG
    a = list(args)
    a[4] = 64 * 16 + 1
    assert lib.s4kv_kivi2_quantize_append(ctypes.byref(good), *a) == s4kv.S4KV_ERR_INVALID_ARG
    a[4] = 0
    assert lib.s4kv_kivi2_quantize_append(ctypes.byref(good), *a) == s4kv.S4KV_OK
    ws = s4kv.s4kv_decode_workspace_bytes(Shape(**GOOD), 1000)

    def call(shape=good, max_ctx=1000, ws_bytes=ws, null_at=None):
        ptrs = [fake] * 6
        if null_at is not None:
            ptrs[null_at] = None
        q, pages, tk, tv, bt, cl = ptrs
        return lib.s4kv_kivi2_paged_decode(ctypes.byref(shape), q, pages, tk, tv, bt, cl, max_ctx,
                                           ctypes.c_float(0.088), fake, fake, ws_bytes, None)

    assert call(shape=bad) == s4kv.S4KV_ERR_UNSUPPORTED
    assert call(max_ctx=0) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(max_ctx=64 * 16 + 1) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(ws_bytes=ws - 1) == s4kv.S4KV_ERR_WORKSPACE
    for i in range(6):
        assert call(null_at=i) == s4kv.S4KV_ERR_INVALID_ARG


def test_mq_workspace_and_refusals():
    sh = Shape(**GOOD)                                   # G = 32 / 8 = 4
    w1 = s4kv.s4kv_mq_workspace_bytes(sh, 1000, 1)
    assert w1 == s4kv.s4kv_decode_workspace_bytes(sh, 1000)   # one token: the decode workspace
    assert s4kv.s4kv_mq_workspace_bytes(sh, 1000, 4) > w1
    # 5 tokens x 4 heads: two column tiles, twice the virtual sequences
    assert s4kv.s4kv_mq_workspace_bytes(sh, 1000, 5) > s4kv.s4kv_mq_workspace_bytes(sh, 1000, 4)
    # 70000 tokens in tiles of 4: more than 65535 virtual sequences
    assert s4kv.s4kv_mq_workspace_bytes(sh, 1000, 70000) == 0
    assert s4kv.s4kv_mq_workspace_bytes(sh, 1000, 0) == 0
    assert s4kv.s4kv_mq_workspace_bytes(sh, 0, 1) == 0
    lib, P, fake = _raw_calls()
    good = Shape(**GOOD).c()
    ws = s4kv.s4kv_mq_workspace_bytes(sh, 1000, 4)

    def call(max_q=4, total_q=16, max_ctx=1000, ws_bytes=ws, null_at=None, shape=good):
        ptrs = [fake] * 9
        if null_at is not None:
            ptrs[null_at] = None
        q, cu, pages, tk, tv, bt, cl, out, wsp = ptrs
        return lib.s4kv_paged_attention_mq(ctypes.byref(shape), q, cu, max_q, total_q, pages, tk, tv,
                                           bt, cl, max_ctx, ctypes.c_float(0.088), out, wsp, ws_bytes,
                                           None)

    assert call(max_q=5) == s4kv.S4KV_ERR_WORKSPACE              # two tiles need more
    assert call(max_q=70000) == s4kv.S4KV_ERR_UNSUPPORTED
    assert call(max_q=0) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(total_q=0) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(total_q=4 * 4 + 1) == s4kv.S4KV_ERR_INVALID_ARG     # more rows than B * max_q
    assert call(max_ctx=0) == s4kv.S4KV_ERR_INVALID_ARG
    assert call(ws_bytes=ws - 1) == s4kv.S4KV_ERR_WORKSPACE
    assert call(shape=Shape(**{**GOOD, "page_size": 8}).c()) == s4kv.S4KV_ERR_UNSUPPORTED
    for i in range(9):
        assert call(null_at=i) == s4kv.S4KV_ERR_INVALID_ARG


def test_check_tables_refuses_before_launch():
    lib, P, fake = _raw_calls()
    good = Shape(**GOOD).c()
    bad = Shape(**{**GOOD, "num_q_heads": 12}).c()
    assert lib.s4kv_check_tables(ctypes.byref(bad), fake, fake, 0, fake, None) == \
        s4kv.S4KV_ERR_UNSUPPORTED
    assert lib.s4kv_check_tables(None, fake, fake, 0, fake, None) == s4kv.S4KV_ERR_INVALID_ARG
    assert lib.s4kv_check_tables(ctypes.byref(good), fake, fake, -1, fake, None) == \
        s4kv.S4KV_ERR_INVALID_ARG
    for null_at in range(3):
        ptrs = [fake] * 3
        ptrs[null_at] = None
        bt, cl, rep = ptrs
        assert lib.s4kv_check_tables(ctypes.byref(good), bt, cl, 1000, rep, None) == \
            s4kv.S4KV_ERR_INVALID_ARG
