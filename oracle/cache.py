"""Logical state of one sequence's paged int4 cache (oracle; test infrastructure only).

PagedAttention explainers (gyaansetu.com "KV-Cache und PagedAttention", section
"Wie PagedAttention das loest"; polaris7.io signal page, "Wichtigste Kernpunkte
& Evidenz") describe a cache cut into fixed-size pages of 16 tokens. The S4 KV
product page ("Funktionsweise" step 1) stores those pages in int4.

Reading taken here (the pages are silent on it): a page is quantized exactly
once, when its 16th token arrives, from the fp16 values of its 16 tokens. The
tokens of the last, not yet full page stay in fp16, K and V alike (the fp16
residual tail). The state therefore depends only on the token values and the
context length, not on how the tokens arrived (one bulk prefill or many
single-token appends): that is what the GPU path is compared with.
"""

import numpy as np

from .quant import flush_pages, dequantize_pages

PAGE = 16


def sequence_cache(k16, v16, bits=4):
    """Cache state of one sequence.

    ``k16``, ``v16``: float16 ``[ctx, Hkv, D]``, the token stream so far.
    ``bits``: code width of the full pages (4, or 2 for the 2-bit variant).

    Returns a dict:
      ``full``  number of int4 pages (ctx // 16),
      ``pages`` output of :func:`flush_pages` with leading dims [full, Hkv],
      ``tail_k``, ``tail_v`` float16 ``[ctx % 16, Hkv, D]``.
    """
    k16 = np.asarray(k16)
    v16 = np.asarray(v16)
    if k16.dtype != np.float16 or v16.dtype != np.float16:
        raise TypeError("K and V must be float16")
    ctx, hkv, d = k16.shape
    full = ctx // PAGE
    kp = k16[: full * PAGE].reshape(full, PAGE, hkv, d).transpose(0, 2, 1, 3)
    vp = v16[: full * PAGE].reshape(full, PAGE, hkv, d).transpose(0, 2, 1, 3)
    pages = flush_pages(np.ascontiguousarray(kp), np.ascontiguousarray(vp), bits)
    return {
        "full": full,
        "pages": pages,
        "tail_k": k16[full * PAGE:].copy(),
        "tail_v": v16[full * PAGE:].copy(),
    }


def dequantized_sequence(cache):
    """K_hat, V_hat as float32 ``[ctx, Hkv, D]``.

    int4 pages are dequantized (code * scale + zero in fp32); tail tokens are
    their exact fp16 values.
    """
    khat_p, vhat_p = dequantize_pages(cache["pages"])  # [full, Hkv, 16, D]
    full = cache["full"]
    hkv, d = khat_p.shape[1], khat_p.shape[3]
    khat = khat_p.transpose(0, 2, 1, 3).reshape(full * PAGE, hkv, d)
    vhat = vhat_p.transpose(0, 2, 1, 3).reshape(full * PAGE, hkv, d)
    khat = np.concatenate([khat, cache["tail_k"].astype(np.float32)], axis=0)
    vhat = np.concatenate([vhat, cache["tail_v"].astype(np.float32)], axis=0)
    return khat, vhat
