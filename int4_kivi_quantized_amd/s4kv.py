"""Thin Python binding of the s4kv C ABI (include/s4kv.h).

Argument marshalling only: every step of quantization and attention runs in
the HIP kernels of libs4kv.so. torch provides device memory and the current
stream. There is no fallback: if the library is missing or a call fails, an
exception is raised.

Function names are the C names; tensor arguments replace the raw pointers and
are checked for dtype, device and contiguity before the call.
"""

import ctypes
import os
from dataclasses import dataclass

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libs4kv.so")

HEAD_DIM = 128
PAGE_SIZE = 16
CHUNK_BYTES = 2624
CHUNK_STRIDE = 2688
MAX_GROUP = 16
F16_CHUNK_BYTES = 8192  # fp16 control pool: K [16][128] then V^T [128][16] per (page, KV head)
FP8_CHUNK_BYTES = 4096  # FP8 pool: E4M3 K and V per (page, KV head), operand order
K2_CHUNK_BYTES = 1600   # 2-bit KIVI pool: data bytes per (page, KV head)
K2_CHUNK_STRIDE = 1664  # and the chunk pitch

S4KV_OK = 0
S4KV_ERR_INVALID_ARG = 1
S4KV_ERR_UNSUPPORTED = 2
S4KV_ERR_WORKSPACE = 3
S4KV_ERR_HIP = 4
S4KV_ERR_SCRATCH_LIMIT = 5
NOALLOC_SCRATCH_BYTES = 32 << 20


class S4KVError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {s4kv_status_string(status)} (status {status})")


class _Shape(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
    ]


@dataclass(frozen=True)
class Shape:
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    num_pages: int
    max_pages_per_seq: int
    head_dim: int = HEAD_DIM
    page_size: int = PAGE_SIZE

    def c(self):
        return _Shape(self.num_seqs, self.num_q_heads, self.num_kv_heads, self.head_dim,
                      self.page_size, self.num_pages, self.max_pages_per_seq)


_lib = None


def library_path():
    return _LIB_PATH


def load():
    """Load libs4kv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m int4_kivi_quantized_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    SP = ctypes.POINTER(_Shape)
    I32 = ctypes.c_int32
    lib.s4kv_validate.argtypes = [SP]
    lib.s4kv_validate.restype = ctypes.c_int
    lib.s4kv_status_string.argtypes = [ctypes.c_int]
    lib.s4kv_status_string.restype = ctypes.c_char_p
    lib.s4kv_pool_bytes.argtypes = [SP]
    lib.s4kv_pool_bytes.restype = ctypes.c_size_t
    lib.s4kv_tail_bytes.argtypes = [SP]
    lib.s4kv_tail_bytes.restype = ctypes.c_size_t
    lib.s4kv_quantize_append.argtypes = [SP, P, P, P, P, I32, P, P, P, P, P]
    lib.s4kv_quantize_append.restype = ctypes.c_int
    lib.s4kv_decode_workspace_bytes.argtypes = [SP, I32]
    lib.s4kv_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.s4kv_paged_decode.argtypes = [SP, P, P, P, P, P, P, I32, ctypes.c_float, P, P,
                                      ctypes.c_size_t, P]
    lib.s4kv_paged_decode.restype = ctypes.c_int
    lib.s4kv_paged_decode_append.argtypes = [SP, P, P, P, P, P, P, P, P, I32, ctypes.c_float, P,
                                             P, ctypes.c_size_t, P]
    lib.s4kv_paged_decode_append.restype = ctypes.c_int
    lib.s4kv_paged_decode_append_noalloc.argtypes = [SP, P, P, P, P, P, P, P, P, I32,
                                                     ctypes.c_float, P, P]
    lib.s4kv_paged_decode_append_noalloc.restype = ctypes.c_int
    lib.s4kv_fp16_pool_bytes.argtypes = [SP]
    lib.s4kv_fp16_pool_bytes.restype = ctypes.c_size_t
    lib.s4kv_fp16_append.argtypes = [SP, P, P, P, P, I32, P, P, P]
    lib.s4kv_fp16_append.restype = ctypes.c_int
    lib.s4kv_fp16_paged_decode.argtypes = [SP, P, P, P, P, I32, ctypes.c_float, P, P,
                                           ctypes.c_size_t, P]
    lib.s4kv_fp16_paged_decode.restype = ctypes.c_int
    lib.s4kv_fp8_pool_bytes.argtypes = [SP]
    lib.s4kv_fp8_pool_bytes.restype = ctypes.c_size_t
    lib.s4kv_fp8_append.argtypes = [SP, P, P, P, P, I32, P, P, P, P, P]
    lib.s4kv_fp8_append.restype = ctypes.c_int
    lib.s4kv_fp8_paged_decode.argtypes = [SP, P, P, P, P, I32, ctypes.c_float, P, P, P, P,
                                          ctypes.c_size_t, P]
    lib.s4kv_fp8_paged_decode.restype = ctypes.c_int
    lib.s4kv_kivi2_pool_bytes.argtypes = [SP]
    lib.s4kv_kivi2_pool_bytes.restype = ctypes.c_size_t
    lib.s4kv_kivi2_quantize_append.argtypes = [SP, P, P, P, P, I32, P, P, P, P, P]
    lib.s4kv_kivi2_quantize_append.restype = ctypes.c_int
    lib.s4kv_kivi2_paged_decode.argtypes = [SP, P, P, P, P, P, P, I32, ctypes.c_float, P, P,
                                            ctypes.c_size_t, P]
    lib.s4kv_kivi2_paged_decode.restype = ctypes.c_int
    lib.s4kv_mq_workspace_bytes.argtypes = [SP, I32, I32]
    lib.s4kv_mq_workspace_bytes.restype = ctypes.c_size_t
    lib.s4kv_paged_attention_mq.argtypes = [SP, P, P, I32, I32, P, P, P, P, P, I32, ctypes.c_float,
                                            P, P, ctypes.c_size_t, P]
    lib.s4kv_paged_attention_mq.restype = ctypes.c_int
    lib.s4kv_check_tables.argtypes = [SP, P, P, I32, P, P]
    lib.s4kv_check_tables.restype = ctypes.c_int
    lib.s4kv_probe_read.argtypes = [P, ctypes.c_size_t, P, I32, I32, I32, P]
    lib.s4kv_probe_read.restype = ctypes.c_int
    _lib = lib
    return lib


EXPORTED = (
    "s4kv_validate", "s4kv_status_string", "s4kv_pool_bytes", "s4kv_tail_bytes",
    "s4kv_quantize_append", "s4kv_decode_workspace_bytes", "s4kv_paged_decode",
    "s4kv_paged_decode_append", "s4kv_paged_decode_append_noalloc",
    "s4kv_fp16_pool_bytes", "s4kv_fp16_append", "s4kv_fp16_paged_decode",
    "s4kv_fp8_pool_bytes", "s4kv_fp8_append", "s4kv_fp8_paged_decode",
    "s4kv_mq_workspace_bytes", "s4kv_paged_attention_mq",
    "s4kv_kivi2_pool_bytes", "s4kv_kivi2_quantize_append", "s4kv_kivi2_paged_decode",
    "s4kv_check_tables", "s4kv_probe_read",
)


def s4kv_status_string(status):
    return load().s4kv_status_string(int(status)).decode()


def s4kv_validate(shape):
    return load().s4kv_validate(ctypes.byref(shape.c()))


def s4kv_pool_bytes(shape):
    return load().s4kv_pool_bytes(ctypes.byref(shape.c()))


def s4kv_tail_bytes(shape):
    return load().s4kv_tail_bytes(ctypes.byref(shape.c()))


def s4kv_decode_workspace_bytes(shape, max_ctx):
    return load().s4kv_decode_workspace_bytes(ctypes.byref(shape.c()), int(max_ctx))


def _ptr(t, dtype, name, device=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _numel(t, want, name, at_least=False):
    """The C ABI sees only pointers: a tensor of the wrong size would make the
    kernels read or write out of bounds, so sizes are checked here."""
    n = t.numel()
    if (n < want) if at_least else (n != want):
        rel = "at least " if at_least else ""
        raise ValueError(f"{name} has {n} elements, needs {rel}{want}")


def _rows(t, row, name):
    """Tensor holding whole rows of ``row`` elements; returns the row count."""
    if t.numel() % row:
        raise ValueError(f"{name} has {t.numel()} elements, not a multiple of {row}")
    return t.numel() // row


def _check_tables(shape, block_table, ctx_lens=None):
    _numel(block_table, shape.num_seqs * shape.max_pages_per_seq, "block_table")
    if ctx_lens is not None:
        _numel(ctx_lens, shape.num_seqs, "ctx_lens")


def _check_tails(shape, tail_k, tail_v):
    n = shape.num_seqs * shape.num_kv_heads * PAGE_SIZE * HEAD_DIM
    _numel(tail_k, n, "tail_k", at_least=True)
    _numel(tail_v, n, "tail_v", at_least=True)


def _check_new_tokens(shape, k, v, cu_new, slot):
    row = shape.num_kv_heads * HEAD_DIM
    if _rows(k, row, "k") != _rows(v, row, "v"):
        raise ValueError("k and v must hold the same number of tokens")
    _numel(cu_new, shape.num_seqs + 1, "cu_new")
    _numel(slot, shape.num_seqs, "slot")


def _check_q_out(shape, q, out):
    _numel(q, shape.num_seqs * shape.num_q_heads * HEAD_DIM, "q")
    _numel(out, shape.num_seqs * shape.num_q_heads * HEAD_DIM, "out")


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status, where):
    if status != S4KV_OK:
        raise S4KVError(status, where)


def s4kv_quantize_append(shape, k, v, cu_new, slot, max_new, block_table, pages, tail_k, tail_v,
                         stream=None):
    """Append new K/V tokens (fp16 [total_new, Hkv, 128]) to every sequence; see s4kv.h."""
    import torch
    _check_new_tokens(shape, k, v, cu_new, slot)
    _check_tables(shape, block_table)
    _numel(pages, s4kv_pool_bytes(shape), "pages", at_least=True)
    _check_tails(shape, tail_k, tail_v)
    st = load().s4kv_quantize_append(
        ctypes.byref(shape.c()), _ptr(k, torch.float16, "k"), _ptr(v, torch.float16, "v"),
        _ptr(cu_new, torch.int32, "cu_new"), _ptr(slot, torch.int32, "slot"), int(max_new),
        _ptr(block_table, torch.int32, "block_table"), _ptr(pages, torch.uint8, "pages"),
        _ptr(tail_k, torch.float16, "tail_k"), _ptr(tail_v, torch.float16, "tail_v"),
        _stream(stream))
    _check(st, "s4kv_quantize_append")


def s4kv_paged_decode(shape, q, pages, tail_k, tail_v, block_table, ctx_lens, max_ctx, sm_scale,
                      out, workspace, stream=None):
    """One decode step: out fp16 [B, Hq, 128] from q fp16 [B, Hq, 128]; see s4kv.h."""
    import torch
    _check_q_out(shape, q, out)
    _check_tables(shape, block_table, ctx_lens)
    _numel(pages, s4kv_pool_bytes(shape), "pages", at_least=True)
    _check_tails(shape, tail_k, tail_v)
    st = load().s4kv_paged_decode(
        ctypes.byref(shape.c()), _ptr(q, torch.float16, "q"), _ptr(pages, torch.uint8, "pages"),
        _ptr(tail_k, torch.float16, "tail_k"), _ptr(tail_v, torch.float16, "tail_v"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(ctx_lens, torch.int32, "ctx_lens"),
        int(max_ctx), float(sm_scale), _ptr(out, torch.float16, "out"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "s4kv_paged_decode")


def s4kv_paged_decode_append(shape, q, k_new, v_new, pages, tail_k, tail_v, block_table, ctx_lens,
                             max_ctx, sm_scale, out, workspace, stream=None):
    """Append one token per sequence (k_new, v_new fp16 [B, Hkv, 128]; ctx_lens
    count it) and decode, in one call; see s4kv.h."""
    import torch
    _check_q_out(shape, q, out)
    _numel(k_new, shape.num_seqs * shape.num_kv_heads * HEAD_DIM, "k_new")
    _numel(v_new, shape.num_seqs * shape.num_kv_heads * HEAD_DIM, "v_new")
    _check_tables(shape, block_table, ctx_lens)
    _numel(pages, s4kv_pool_bytes(shape), "pages", at_least=True)
    _check_tails(shape, tail_k, tail_v)
    st = load().s4kv_paged_decode_append(
        ctypes.byref(shape.c()), _ptr(q, torch.float16, "q"), _ptr(k_new, torch.float16, "k_new"),
        _ptr(v_new, torch.float16, "v_new"), _ptr(pages, torch.uint8, "pages"),
        _ptr(tail_k, torch.float16, "tail_k"), _ptr(tail_v, torch.float16, "tail_v"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(ctx_lens, torch.int32, "ctx_lens"),
        int(max_ctx), float(sm_scale), _ptr(out, torch.float16, "out"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "s4kv_paged_decode_append")


def s4kv_paged_decode_append_noalloc(shape, q, k_new, v_new, pages, tail_k, tail_v, block_table,
                                     ctx_lens, max_ctx, sm_scale, out, stream=None):
    """s4kv_paged_decode_append with the decode workspace in the library's
    static per-device array (no workspace argument, nothing allocated); see
    s4kv.h."""
    import torch
    _check_q_out(shape, q, out)
    _numel(k_new, shape.num_seqs * shape.num_kv_heads * HEAD_DIM, "k_new")
    _numel(v_new, shape.num_seqs * shape.num_kv_heads * HEAD_DIM, "v_new")
    _check_tables(shape, block_table, ctx_lens)
    _numel(pages, s4kv_pool_bytes(shape), "pages", at_least=True)
    _check_tails(shape, tail_k, tail_v)
    st = load().s4kv_paged_decode_append_noalloc(
        ctypes.byref(shape.c()), _ptr(q, torch.float16, "q"), _ptr(k_new, torch.float16, "k_new"),
        _ptr(v_new, torch.float16, "v_new"), _ptr(pages, torch.uint8, "pages"),
        _ptr(tail_k, torch.float16, "tail_k"), _ptr(tail_v, torch.float16, "tail_v"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(ctx_lens, torch.int32, "ctx_lens"),
        int(max_ctx), float(sm_scale), _ptr(out, torch.float16, "out"), _stream(stream))
    _check(st, "s4kv_paged_decode_append_noalloc")


def s4kv_mq_workspace_bytes(shape, max_ctx, max_q):
    return load().s4kv_mq_workspace_bytes(ctypes.byref(shape.c()), int(max_ctx), int(max_q))


def s4kv_paged_attention_mq(shape, q, cu_q, max_q, pages, tail_k, tail_v, block_table, ctx_lens,
                            max_ctx, sm_scale, out, workspace, stream=None):
    """Multi-query attention: out fp16 [total_q, Hq, 128] from q fp16 [total_q, Hq, 128], the
    rows of sequence b being cu_q[b] .. cu_q[b+1]-1 (int32 [B+1]); see s4kv.h."""
    import torch
    _rows(q, shape.num_q_heads * HEAD_DIM, "q")
    _numel(out, q.numel(), "out")
    _numel(cu_q, shape.num_seqs + 1, "cu_q")
    _check_tables(shape, block_table, ctx_lens)
    _numel(pages, s4kv_pool_bytes(shape), "pages", at_least=True)
    _check_tails(shape, tail_k, tail_v)
    st = load().s4kv_paged_attention_mq(
        ctypes.byref(shape.c()), _ptr(q, torch.float16, "q"), _ptr(cu_q, torch.int32, "cu_q"),
        int(max_q), int(q.shape[0]), _ptr(pages, torch.uint8, "pages"),
        _ptr(tail_k, torch.float16, "tail_k"), _ptr(tail_v, torch.float16, "tail_v"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(ctx_lens, torch.int32, "ctx_lens"),
        int(max_ctx), float(sm_scale), _ptr(out, torch.float16, "out"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "s4kv_paged_attention_mq")


def s4kv_check_tables(shape, block_table, ctx_lens, max_ctx, report, stream=None):
    """Check block_table / ctx_lens against the shape on the device; report int32 [4] is
    written (fault counts, first faulty sequence and page); see s4kv.h."""
    import torch
    _check_tables(shape, block_table, ctx_lens)
    _numel(report, 4, "report")
    st = load().s4kv_check_tables(
        ctypes.byref(shape.c()), _ptr(block_table, torch.int32, "block_table"),
        _ptr(ctx_lens, torch.int32, "ctx_lens"), int(max_ctx), _ptr(report, torch.int32, "report"),
        _stream(stream))
    _check(st, "s4kv_check_tables")


def s4kv_fp16_pool_bytes(shape):
    return load().s4kv_fp16_pool_bytes(ctypes.byref(shape.c()))


def s4kv_fp16_append(shape, k, v, cu_new, slot, max_new, block_table, pages, stream=None):
    """Append new K/V tokens (fp16 [total_new, Hkv, 128]) to the fp16 pool; see s4kv.h."""
    import torch
    _check_new_tokens(shape, k, v, cu_new, slot)
    _check_tables(shape, block_table)
    _numel(pages, s4kv_fp16_pool_bytes(shape) // 2, "pages", at_least=True)
    st = load().s4kv_fp16_append(
        ctypes.byref(shape.c()), _ptr(k, torch.float16, "k"), _ptr(v, torch.float16, "v"),
        _ptr(cu_new, torch.int32, "cu_new"), _ptr(slot, torch.int32, "slot"), int(max_new),
        _ptr(block_table, torch.int32, "block_table"), _ptr(pages, torch.float16, "pages"),
        _stream(stream))
    _check(st, "s4kv_fp16_append")


def s4kv_fp16_paged_decode(shape, q, pages, block_table, ctx_lens, max_ctx, sm_scale, out,
                           workspace, stream=None):
    """One decode step over the fp16 pool: out fp16 [B, Hq, 128]; see s4kv.h."""
    import torch
    _check_q_out(shape, q, out)
    _check_tables(shape, block_table, ctx_lens)
    _numel(pages, s4kv_fp16_pool_bytes(shape) // 2, "pages", at_least=True)
    st = load().s4kv_fp16_paged_decode(
        ctypes.byref(shape.c()), _ptr(q, torch.float16, "q"), _ptr(pages, torch.float16, "pages"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(ctx_lens, torch.int32, "ctx_lens"),
        int(max_ctx), float(sm_scale), _ptr(out, torch.float16, "out"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "s4kv_fp16_paged_decode")


def s4kv_fp8_pool_bytes(shape):
    return load().s4kv_fp8_pool_bytes(ctypes.byref(shape.c()))


def s4kv_fp8_append(shape, k, v, cu_new, slot, max_new, block_table, k_scale, v_scale, pages,
                    stream=None):
    """Quantize new K/V tokens (fp16 [total_new, Hkv, 128]) to E4M3 with the per-KV-head
    scales (fp32 [Hkv]) and append them to the FP8 pool; see s4kv.h."""
    import torch
    _check_new_tokens(shape, k, v, cu_new, slot)
    _check_tables(shape, block_table)
    _numel(k_scale, shape.num_kv_heads, "k_scale")
    _numel(v_scale, shape.num_kv_heads, "v_scale")
    _numel(pages, s4kv_fp8_pool_bytes(shape), "pages", at_least=True)
    st = load().s4kv_fp8_append(
        ctypes.byref(shape.c()), _ptr(k, torch.float16, "k"), _ptr(v, torch.float16, "v"),
        _ptr(cu_new, torch.int32, "cu_new"), _ptr(slot, torch.int32, "slot"), int(max_new),
        _ptr(block_table, torch.int32, "block_table"), _ptr(k_scale, torch.float32, "k_scale"),
        _ptr(v_scale, torch.float32, "v_scale"), _ptr(pages, torch.uint8, "pages"),
        _stream(stream))
    _check(st, "s4kv_fp8_append")


def s4kv_fp8_paged_decode(shape, q, pages, block_table, ctx_lens, max_ctx, sm_scale, k_scale,
                          v_scale, out, workspace, stream=None):
    """One decode step over the FP8 pool: out fp16 [B, Hq, 128]; see s4kv.h."""
    import torch
    _check_q_out(shape, q, out)
    _check_tables(shape, block_table, ctx_lens)
    _numel(k_scale, shape.num_kv_heads, "k_scale")
    _numel(v_scale, shape.num_kv_heads, "v_scale")
    _numel(pages, s4kv_fp8_pool_bytes(shape), "pages", at_least=True)
    st = load().s4kv_fp8_paged_decode(
        ctypes.byref(shape.c()), _ptr(q, torch.float16, "q"), _ptr(pages, torch.uint8, "pages"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(ctx_lens, torch.int32, "ctx_lens"),
        int(max_ctx), float(sm_scale), _ptr(k_scale, torch.float32, "k_scale"),
        _ptr(v_scale, torch.float32, "v_scale"), _ptr(out, torch.float16, "out"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "s4kv_fp8_paged_decode")


def s4kv_probe_read(pool, chunk_ids, chunks_per_wave, waves, non_temporal=True, stream=None):
    """Read 4096-byte chunks of pool (uint8) with the decode kernels' load path;
    a measurement aid, see include/s4kv_probe.h."""
    import torch
    st = load().s4kv_probe_read(
        _ptr(pool, torch.uint8, "pool"), pool.numel(), _ptr(chunk_ids, torch.int32, "chunk_ids"),
        int(chunks_per_wave), int(waves), 1 if non_temporal else 0, _stream(stream))
    _check(st, "s4kv_probe_read")


def s4kv_kivi2_pool_bytes(shape):
    return load().s4kv_kivi2_pool_bytes(ctypes.byref(shape.c()))


def s4kv_kivi2_quantize_append(shape, k, v, cu_new, slot, max_new, block_table, pages, tail_k,
                               tail_v, stream=None):
    """s4kv_quantize_append with 2-bit codes into the 2-bit pool; see s4kv.h."""
    import torch
    _check_new_tokens(shape, k, v, cu_new, slot)
    _check_tables(shape, block_table)
    _numel(pages, s4kv_kivi2_pool_bytes(shape), "pages", at_least=True)
    _check_tails(shape, tail_k, tail_v)
    st = load().s4kv_kivi2_quantize_append(
        ctypes.byref(shape.c()), _ptr(k, torch.float16, "k"), _ptr(v, torch.float16, "v"),
        _ptr(cu_new, torch.int32, "cu_new"), _ptr(slot, torch.int32, "slot"), int(max_new),
        _ptr(block_table, torch.int32, "block_table"), _ptr(pages, torch.uint8, "pages"),
        _ptr(tail_k, torch.float16, "tail_k"), _ptr(tail_v, torch.float16, "tail_v"),
        _stream(stream))
    _check(st, "s4kv_kivi2_quantize_append")


def s4kv_kivi2_paged_decode(shape, q, pages, tail_k, tail_v, block_table, ctx_lens, max_ctx,
                            sm_scale, out, workspace, stream=None):
    """s4kv_paged_decode over the 2-bit pool; see s4kv.h."""
    import torch
    _check_q_out(shape, q, out)
    _check_tables(shape, block_table, ctx_lens)
    _numel(pages, s4kv_kivi2_pool_bytes(shape), "pages", at_least=True)
    _check_tails(shape, tail_k, tail_v)
    st = load().s4kv_kivi2_paged_decode(
        ctypes.byref(shape.c()), _ptr(q, torch.float16, "q"), _ptr(pages, torch.uint8, "pages"),
        _ptr(tail_k, torch.float16, "tail_k"), _ptr(tail_v, torch.float16, "tail_v"),
        _ptr(block_table, torch.int32, "block_table"), _ptr(ctx_lens, torch.int32, "ctx_lens"),
        int(max_ctx), float(sm_scale), _ptr(out, torch.float16, "out"),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check(st, "s4kv_kivi2_paged_decode")
