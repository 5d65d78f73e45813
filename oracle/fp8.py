"""FP8 (E4M3) KV cache with per-KV-head scales (oracle; test infrastructure only).

The FP8 KV cache is the quantized-KV variant the pages discuss most: the
KV-quantization guide on adechristanto.de (sections "Der Eingriff kann
Attention-Arithmetik einschliessen" and the one after it) describes vLLM's FP8
KV cache with default scales of 1.0 or calibrated scales, per tensor or per
attention head; the polaris7.io signal page ("Wichtigste Kernpunkte &
Evidenz") names the `--kv-cache-dtype fp8` switch, and the reference list of
the analyticslegends.ai page names the fp8_e4m3 / fp8_e5m2 cache dtypes.

Readings taken here (the pages fix no formula):

1. element format: OCP FP8 E4M3 -- 1 sign bit, 4 exponent bits (bias 7),
   3 mantissa bits, subnormals below 2^-6 with step 2^-9, largest finite
   value 448, no infinities, NaN = S.1111.111;
2. one fp32 scale per KV head for K and one for V (a per-tensor scale is the
   case of equal values); q stays fp16 (the guide notes that some backends
   also quantize queries; this path does not);
3. encode: y = fp32(x) / fp32(scale) as one IEEE fp32 division, then
   round to nearest E4M3 value with ties to even; magnitudes of 448 and more
   saturate to 448; the sign of y is kept, also for a zero result;
4. decode: value(code) * scale.

Written from the format definition; shares nothing with the HIP library.
"""

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code):
    """float64 value of E4M3 codes (uint8 array-like); NaN for S.1111.111."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(y32):
    """E4M3 codes (uint8) of float32 values: round to nearest, ties to even,
    saturating at 448 (reading 3). NaN inputs are out of contract."""
    y = np.asarray(y32, dtype=np.float32)
    sign = np.where(np.signbit(y), 0x80, 0).astype(np.int64)
    a = np.abs(y).astype(np.float64)           # exact: every step below is exact in fp32 too
    out = np.zeros(y.shape, dtype=np.int64)
    sat = a >= E4M3_MAX
    sub = a < 2.0 ** -6
    nrm = ~sat & ~sub
    # subnormal range: multiples of 2^-9; 8 * 2^-9 is the smallest normal (code 8)
    out[sub] = np.rint(a[sub] * 512.0).astype(np.int64)
    # normal range: a = f * 2^k with f in [0.5, 1), so a = (2f) * 2^(k-1)
    f, k = np.frexp(a[nrm])
    e = k - 1
    mant = np.rint((2.0 * f - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8
    mant = np.where(carry, 0, mant)
    e = np.where(carry, e + 1, e)
    out[nrm] = np.minimum(((e + 7) << 3) | mant, 0x7E)
    out[sat] = 0x7E
    return (sign | out).astype(np.uint8)


def quantize_fp8(x16, scale):
    """Codes of fp16 values x16 (any shape) with one fp32 scale (reading 3)."""
    y = np.asarray(x16, dtype=np.float16).astype(np.float32) / np.float32(scale)
    return e4m3_encode(y)


def fp8_sequence(k16, v16, k_scale, v_scale):
    """One sequence's FP8 cache: codes [ctx, Hkv, D] of K and V, each KV head
    h quantized with k_scale[h] / v_scale[h]."""
    k16 = np.asarray(k16, dtype=np.float16)
    v16 = np.asarray(v16, dtype=np.float16)
    hkv = k16.shape[1]
    kc = np.stack([quantize_fp8(k16[:, h], k_scale[h]) for h in range(hkv)], axis=1)
    vc = np.stack([quantize_fp8(v16[:, h], v_scale[h]) for h in range(hkv)], axis=1)
    return kc, vc


def fp8_dequantized(kc, vc, k_scale, v_scale):
    """K_hat, V_hat float64 [ctx, Hkv, D]: code value times the head's scale."""
    ks = np.asarray(k_scale, dtype=np.float64)[None, :, None]
    vs = np.asarray(v_scale, dtype=np.float64)[None, :, None]
    return e4m3_value(kc) * ks, e4m3_value(vc) * vs
