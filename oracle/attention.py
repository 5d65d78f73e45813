"""Decode-time attention over the dequantized cache (oracle; test infrastructure only).

The S4 KV product page (header paragraph, "FAQ" on supported models) names
standard attention with head_dim 128. The KV-cache explainer (analyticslegends.ai,
"Begriffe", entry "Grouped-Query Attention (GQA)") describes groups of query
heads sharing one K/V head.

Readings taken here:
* query head j reads KV head floor(j / G), G = Hq / Hkv (consecutive query
  heads share a KV head);
* logits are sm_scale * q . k_hat with sm_scale = 1 / sqrt(head_dim) by default;
* softmax over all cached tokens, output = sum_t p_t v_hat_t.

The oracle evaluates this in float64 over the fp32 dequantized cache, the
plain definition with no blocking, splitting or reordering.

Several query tokens per sequence (the prefill side of the two inference
phases, named on the polaris7.io signal page, "Verwandte Marktsignale &
Trends", entry on KV caching; also the verify step of speculative decoding):
the new tokens are already in the cache, the last T of its ctx positions, and
token t (position ctx - T + t) attends causally to positions 0 .. ctx - T + t
(reading: causal attention with the new tokens at the end of the cache).
"""

import math

import numpy as np


def decode_attention(q16, khat, vhat, sm_scale=None):
    """One decode step for one sequence.

    ``q16``: [Hq, D] (float16), ``khat``/``vhat``: [ctx, Hkv, D] (float32).
    Returns float64 [Hq, D].
    """
    q = np.asarray(q16).astype(np.float64)
    k = np.asarray(khat).astype(np.float64)
    v = np.asarray(vhat).astype(np.float64)
    hq, d = q.shape
    ctx, hkv, d2 = k.shape
    if d2 != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if ctx < 1:
        raise ValueError("decode needs at least one cached token")
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = hq // hkv
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    out = np.empty((hq, d), dtype=np.float64)
    for j in range(hq):
        h = j // g
        logits = sm_scale * (k[:, h, :] @ q[j])
        m = logits.max()
        p = np.exp(logits - m)
        out[j] = (p @ v[:, h, :]) / p.sum()
    return out


def decode_attention_batch(q16, seq_khat, seq_vhat, sm_scale=None):
    """:func:`decode_attention` for each sequence; lists of per-sequence caches."""
    return [decode_attention(q16[b], seq_khat[b], seq_vhat[b], sm_scale)
            for b in range(len(seq_khat))]


def multiquery_attention(q16, khat, vhat, sm_scale=None):
    """Causal attention of the last T cache positions' queries.

    ``q16``: [T, Hq, D] queries of the tokens at positions ctx - T .. ctx - 1;
    ``khat``/``vhat``: [ctx, Hkv, D]. Token t sees positions 0 .. ctx - T + t.
    Returns float64 [T, Hq, D].
    """
    q = np.asarray(q16)
    ctx = np.asarray(khat).shape[0]
    t_new = q.shape[0]
    if not 1 <= t_new <= ctx:
        raise ValueError("need 1 <= T <= ctx")
    return np.stack([decode_attention(q[t], khat[:ctx - t_new + t + 1], vhat[:ctx - t_new + t + 1],
                                      sm_scale) for t in range(t_new)])
