"""Crafted fp16 K/V pages that hit the quantizer's special cases (test
infrastructure: an input generator, no quantizer or attention arithmetic).

The rule the pages are checked against is the asymmetric min/scale code of the
S4 KV product page (header paragraph and "Funktionsweise" step 1), KEY
grouped per channel over a page's 16 tokens, VALUE per token over its 128
channels. Each page gets, besides seeded N(0, 1) values:

* K channels / V tokens whose group is uniform (scale +0, codes 0), among
  them subnormal, -0 and mixed +-0 groups;
* groups whose minimum is -0 (the zero point must be stored as +0);
* groups whose range underflows the fp16 scale (2^-24 over 15 or 3 rounds
  to 0);
* groups whose scale rounds to a subnormal below (max - min) / qmax, so the
  maximum's quotient exceeds qmax and must clamp (22 * 2^-24 for int4,
  7 * 2^-24 for 2 bits);
* exact-tie grids at unit scale (min 0, max 15, or max 3 for 2 bits, with
  values at half steps: round half to even);
* with ``extreme``: groups at the ends of the fp16 range (+-65504).
"""

import numpy as np

F16 = np.float16
TINY = 2.0 ** -24          # smallest fp16 subnormal


def _full(x):
    return [x] * 16


def special_groups(extreme):
    """16-value groups (lists of floats, each exactly representable in fp16)."""
    g = [
        _full(0.0), _full(1.5), _full(-3.25), _full(6 * TINY), _full(TINY), _full(-0.0),
        [-0.0, 0.0] * 8,                                     # +-0 only: scale +0, zero +0
        [-0.0, 1.0, 2.0, 0.5] * 4,                           # minimum -0
        [0.0, 0.25, -0.0, 3.0] * 4,                          # minimum -0 beside +0
        [0.0] * 8 + [TINY] * 8,                              # range 2^-24: scale underflows
        [0.0] * 15 + [22 * TINY],                            # int4: subnormal scale, clamp at 15
        [0.0] * 15 + [7 * TINY],                             # 2-bit: subnormal scale, clamp at 3
        [-5 * TINY] * 15 + [17 * TINY],                      # subnormal range around zero
        [0, 15, 2.5, 3.5, 0.5, 1.5, 4.5, 13.5, 14.5, 7.25, 7.75, 5.5, 6.5, 8.5, 9.5, 10.5],
        [0, 3, 0.5, 1.5, 2.5, 1.0, 2.0, 0.25, 0.75, 1.25, 1.75, 2.25, 2.75, 0.5, 1.5, 2.5],
        [-8, 7, -7.5, -6.5, -5.5, 6.5, 5.5, 0.5, -0.5, -1.5, 1.5, 2.5, -2.5, 3.5, -3.5, 4.5],
    ]
    if extreme:
        g += [
            _full(65504.0), _full(-65504.0),
            [-65504.0, 65504.0] * 8,
            [-65504.0] * 15 + [65504.0],
            [65504.0, 65472.0, 65440.0, 32768.0] * 4,
            [-65504.0, -0.0, 2048.0, 65504.0] * 4,
        ]
    return [np.asarray(x, dtype=np.float64) for x in g]


def edge_pages(n_pages, hkv, seed, extreme=False, d=128):
    """fp16 K, V [16 * n_pages, hkv, d]: every page of every head carries all
    special groups, at seeded channels (K) and tokens (V); the rest is N(0,1)."""
    rng = np.random.default_rng(seed)
    groups = special_groups(extreme)
    k = rng.standard_normal((n_pages, 16, hkv, d)).astype(F16)
    v = rng.standard_normal((n_pages, 16, hkv, d)).astype(F16)
    for p in range(n_pages):
        for h in range(hkv):
            chans = rng.choice(d, size=len(groups), replace=False)
            for grp, ch in zip(groups, chans):
                k[p, :, h, ch] = rng.permutation(grp).astype(F16)
            # V groups run over the channels: a 16-value pattern tiled 8 times,
            # shuffled, on one token each (16 of the groups per page, chosen
            # at random)
            toks = rng.permutation(16)
            for i, gi in enumerate(rng.choice(len(groups), size=16, replace=False)):
                v[p, toks[i], h, :] = rng.permutation(np.tile(groups[gi], d // 16)).astype(F16)
    return k.reshape(16 * n_pages, hkv, d), v.reshape(16 * n_pages, hkv, d)


def edge_tail(n, hkv, seed, d=128):
    """fp16 K, V [n, hkv, d] of tail tokens (kept in fp16): random with a few
    special values."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, hkv, d)).astype(F16)
    v = rng.standard_normal((n, hkv, d)).astype(F16)
    for x in (k, v):
        flat = x.reshape(-1)
        idx = rng.choice(flat.size, size=min(8, flat.size), replace=False)
        flat[idx] = np.array([-0.0, 0.0, TINY, -TINY, 6 * TINY, 1.5, -3.25, 0.5], F16)[:len(idx)]
    return k, v
