"""The Python binding refuses mis-sized tensors before calling the C ABI,
which sees only pointers (a wrong size would otherwise make a kernel read or
write out of bounds). CPU tensors suffice: the size checks come before the
device check, and no call reaches the library's kernels."""

import pytest
import torch

from int4_kivi_quantized_amd import s4kv
from int4_kivi_quantized_amd.s4kv import Shape

SH = Shape(num_seqs=3, num_q_heads=8, num_kv_heads=2, num_pages=20, max_pages_per_seq=6)
B, HQ, HKV, D = 3, 8, 2, 128


def _t(n, dtype=torch.float16):
    return torch.zeros(n, dtype=dtype)


def _decode_args(**over):
    a = dict(q=_t(B * HQ * D), pages=_t(s4kv.s4kv_pool_bytes(SH), torch.uint8),
             tail_k=_t(B * HKV * 16 * D), tail_v=_t(B * HKV * 16 * D),
             block_table=_t(B * 6, torch.int32), ctx_lens=_t(B, torch.int32),
             out=_t(B * HQ * D), workspace=_t(1 << 20, torch.uint8))
    a.update(over)
    return a


@pytest.mark.parametrize("name,bad", [
    ("q", _t(B * HQ * D - 1)), ("out", _t(B * HQ * D + 128)),
    ("block_table", _t(B * 6 - 1, torch.int32)), ("ctx_lens", _t(B + 1, torch.int32)),
    ("pages", _t(100, torch.uint8)), ("tail_k", _t(16)), ("tail_v", _t(16)),
])
def test_decode_refuses_wrong_sizes(name, bad):
    a = _decode_args(**{name: bad})
    with pytest.raises(ValueError, match=name):
        s4kv.s4kv_paged_decode(SH, a["q"], a["pages"], a["tail_k"], a["tail_v"], a["block_table"],
                               a["ctx_lens"], 64, 0.1, a["out"], a["workspace"])


def test_decode_append_refuses_wrong_new_token_sizes():
    a = _decode_args()
    for name in ("k_new", "v_new"):
        kv = {"k_new": _t(B * HKV * D), "v_new": _t(B * HKV * D)}
        kv[name] = _t(B * HKV * D - 2)
        with pytest.raises(ValueError, match=name):
            s4kv.s4kv_paged_decode_append(SH, a["q"], kv["k_new"], kv["v_new"], a["pages"],
                                          a["tail_k"], a["tail_v"], a["block_table"],
                                          a["ctx_lens"], 64, 0.1, a["out"], a["workspace"])


def test_append_refuses_wrong_sizes():
    a = _decode_args()
    k, v = _t(5 * HKV * D), _t(5 * HKV * D)
    cu, slot = _t(B + 1, torch.int32), _t(B, torch.int32)
    for kw, pat in (({"k": _t(5 * HKV * D + 1)}, "k has"), ({"v": _t(4 * HKV * D)}, "same number"),
                    ({"cu_new": _t(B, torch.int32)}, "cu_new"), ({"slot": _t(B + 1, torch.int32)}, "slot")):
        args = dict(k=k, v=v, cu_new=cu, slot=slot)
        args.update(kw)
        with pytest.raises(ValueError, match=pat):
            s4kv.s4kv_quantize_append(SH, args["k"], args["v"], args["cu_new"], args["slot"], 5,
                                      a["block_table"], a["pages"], a["tail_k"], a["tail_v"])


def test_multiquery_and_dense_refuse_wrong_sizes():
    a = _decode_args()
    q = _t(7 * HQ * D)
    with pytest.raises(ValueError, match="out"):
        s4kv.s4kv_paged_attention_mq(SH, q, _t(B + 1, torch.int32), 2, a["pages"], a["tail_k"],
                                     a["tail_v"], a["block_table"], a["ctx_lens"], 64, 0.1,
                                     _t(6 * HQ * D), a["workspace"])
    with pytest.raises(ValueError, match="cu_q"):
        s4kv.s4kv_paged_attention_mq(SH, q, _t(B, torch.int32), 2, a["pages"], a["tail_k"],
                                     a["tail_v"], a["block_table"], a["ctx_lens"], 64, 0.1,
                                     _t(7 * HQ * D), a["workspace"])
    f16_pages = _t(s4kv.s4kv_fp16_pool_bytes(SH) // 2 - 1)
    with pytest.raises(ValueError, match="pages"):
        s4kv.s4kv_fp16_paged_decode(SH, a["q"], f16_pages, a["block_table"], a["ctx_lens"], 64,
                                    0.1, a["out"], a["workspace"])
    f8_pages = _t(s4kv.s4kv_fp8_pool_bytes(SH), torch.uint8)
    with pytest.raises(ValueError, match="k_scale"):
        s4kv.s4kv_fp8_paged_decode(SH, a["q"], f8_pages, a["block_table"], a["ctx_lens"], 64, 0.1,
                                   _t(HKV + 1, torch.float32), _t(HKV, torch.float32), a["out"],
                                   a["workspace"])


def test_right_sizes_reach_the_device_check():
    """With every size right, the next refusal is the device check (CPU tensors)."""
    a = _decode_args()
    with pytest.raises(ValueError, match="GPU tensor"):
        s4kv.s4kv_paged_decode(SH, a["q"], a["pages"], a["tail_k"], a["tail_v"], a["block_table"],
                               a["ctx_lens"], 64, 0.1, a["out"], a["workspace"])
