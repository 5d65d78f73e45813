"""Asymmetric int4 group quantizer (oracle; test infrastructure only).

Follows the S4 KV product page (abyo.net/de/s4/s4-kv), header paragraph and
"Funktionsweise" step 1: the KV cache is stored in int4, asymmetric, KIVI
style, with KEY grouped per channel and VALUE grouped per token.

The pages give no formula. The readings taken here (each one is listed with
its reason in the design notes) are:

1. zero point = the group minimum, kept as an fp16 value (float zero point);
2. scale = (max - min) / 15 evaluated in fp32 and rounded to fp16 (codes span
   0..15);
3. codes are computed from the *stored* fp16 scale and zero, so that the
   reconstruction error is at most half a stored step;
4. arithmetic is IEEE fp32 with round-to-nearest-even: one subtraction, one
   correctly rounded division (no reciprocal, no fused multiply-add), then
   rounding to the nearest integer with ties to even, then clamping to [0, 15];
5. a group whose fp16 scale is zero (all values equal, or a range so small
   that (max - min) / 15 underflows fp16) gets all codes 0 and dequantizes to
   the zero point exactly;
6. a negative-zero scale or zero point is stored as +0.

Dequantization is x_hat = code * scale + zero in fp32.

The same rule with 2-bit codes (scale = (max - min) / 3, codes 0..3) is the
KIVI variant the KV-cache explainer cites (analyticslegends.ai, "Quellen",
entry 17: KIVI, a tuning-free asymmetric 2-bit quantization of the KV cache):
``bits=2`` replaces 15 by 3 in readings 2 and 4, everything else unchanged.
"""

import numpy as np

QMAX = 15
_F32 = np.float32
_F16 = np.float16


def qmax_of(bits):
    """Largest code of a ``bits``-wide unsigned code (4 -> 15, 2 -> 3)."""
    if bits not in (2, 4):
        raise ValueError("codes are 4 or 2 bits wide")
    return (1 << bits) - 1


def quantize_groups(x16, axis=-1, bits=4):
    """Quantize fp16 groups lying along ``axis``.

    Parameters
    ----------
    x16 : ndarray of float16. Each 1-D slice along ``axis`` is one group.
    axis : the group axis.
    bits : code width, 4 (codes 0..15) or 2 (codes 0..3).

    Returns
    -------
    codes : uint8 array, same shape as ``x16``, values in 0..qmax.
    scale : float16 array, ``x16`` with ``axis`` removed.
    zero  : float16 array, same shape as ``scale``.
    """
    qmax = qmax_of(bits)
    x16 = np.asarray(x16)
    if x16.dtype != _F16:
        raise TypeError("quantize_groups expects float16 input")
    xg = np.moveaxis(x16, axis, -1)
    # Reading 1: the group extremes are fp16 values, compared exactly.
    mn = xg.min(axis=-1)
    mx = xg.max(axis=-1)
    # Reading 2 and 4: fp32 range, fp32 division by qmax, round to fp16 (RNE).
    s32 = (mx.astype(_F32) - mn.astype(_F32)) / _F32(qmax)
    s16 = s32.astype(_F16)
    z16 = mn.astype(_F16)
    # Reading 6: canonical +0.
    s16 = np.where(s16 == 0, _F16(0.0), s16).astype(_F16)
    z16 = np.where(z16 == 0, _F16(0.0), z16).astype(_F16)
    # Reading 3 and 4: codes from the stored fp16 scale/zero, IEEE fp32
    # subtract then divide, round half to even, clamp.
    zero_scale = s16 == 0
    denom = np.where(zero_scale, _F32(1.0), s16.astype(_F32)).astype(_F32)
    t = (xg.astype(_F32) - z16.astype(_F32)[..., None]) / denom[..., None]
    q = np.clip(np.rint(t), 0, qmax)
    # Reading 5: a zero scale gives all-zero codes.
    q = np.where(zero_scale[..., None], _F32(0.0), q)
    codes = np.moveaxis(q.astype(np.uint8), -1, axis)
    return codes, s16, z16


def dequantize(codes, scale, zero, axis=-1):
    """x_hat = code * scale + zero in fp32; ``scale``/``zero`` lack ``axis``."""
    c = np.moveaxis(np.asarray(codes), axis, -1).astype(_F32)
    s = np.asarray(scale).astype(_F32)[..., None]
    z = np.asarray(zero).astype(_F32)[..., None]
    x = c * s + z
    return np.moveaxis(x.astype(_F32), -1, axis)


def flush_pages(k16, v16, bits=4):
    """Quantize full 16-token pages.

    ``k16``, ``v16``: float16 arrays ``[..., 16, D]`` (token, channel) holding
    the 16 tokens of each page for one KV head.

    KEY: one group per channel over the page's 16 tokens (per-channel KEY; the
    group boundary is the page, reading 9 of the design notes).
    VALUE: one group per token over its D channels (per-token VALUE).

    Returns a dict with
      ``ck`` uint8 [..., 16, D], ``sk``/``zk`` float16 [..., D],
      ``cv`` uint8 [..., 16, D], ``sv``/``zv`` float16 [..., 16].
    """
    k16 = np.asarray(k16)
    v16 = np.asarray(v16)
    if k16.shape != v16.shape or k16.shape[-2] != 16:
        raise ValueError("pages must be [..., 16, D] for K and V alike")
    ck, sk, zk = quantize_groups(k16, axis=-2, bits=bits)
    cv, sv, zv = quantize_groups(v16, axis=-1, bits=bits)
    return {"ck": ck, "sk": sk, "zk": zk, "cv": cv, "sv": sv, "zv": zv}


def dequantize_pages(page):
    """Inverse of :func:`flush_pages` up to quantization error (fp32)."""
    khat = dequantize(page["ck"], page["sk"], page["zk"], axis=-2)
    vhat = dequantize(page["cv"], page["sv"], page["zv"], axis=-1)
    return khat, vhat
