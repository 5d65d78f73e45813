"""int4 KIVI paged KV cache for AMD Instinct MI355X (gfx950).

The compute lives in libs4kv.so (hand-written HIP kernels behind the C ABI in
include/s4kv.h); ``s4kv`` is its thin Python binding and ``cache`` holds
device-side buffers for one layer.
"""

from . import s4kv  # noqa: F401
from .s4kv import (  # noqa: F401
    Shape,
    S4KVError,
    s4kv_validate,
    s4kv_status_string,
    s4kv_pool_bytes,
    s4kv_tail_bytes,
    s4kv_quantize_append,
    s4kv_decode_workspace_bytes,
    s4kv_paged_decode,
)
