"""The host replica of the decode stream's work split (tests/unit_split.py),
which the GPU tests use to know which kernel route a case exercises, checked
against a unit-by-unit walk of the same rules on random small cases."""

import numpy as np

from tests.unit_split import completion_kinds, walk_entries


def _kinds_from_walk(ctx, hkv, waves):
    pair_b = single = 0
    for _, b, h, unit, n in walk_entries(ctx, hkv, waves):
        if n and ctx[b] > 0 and ctx[b] % 16 == 0 and unit + n == ctx[b] // 16:
            if n == 2:
                pair_b += 1
            else:
                single += 1
    return pair_b, single


def test_completion_kinds_match_walk():
    rng = np.random.default_rng(0)
    for _ in range(60):
        b = int(rng.integers(1, 20))
        hkv = int(rng.integers(1, 4))
        waves = int(rng.integers(1, 64))
        ctx = rng.integers(0, 200, size=b)
        ctx[rng.integers(0, b)] = 16 * int(rng.integers(1, 12))   # at least one completion
        assert completion_kinds(ctx, hkv, waves) == _kinds_from_walk(ctx, hkv, waves)


def test_walk_covers_every_unit_once():
    rng = np.random.default_rng(1)
    for _ in range(30):
        b = int(rng.integers(1, 12))
        hkv = int(rng.integers(1, 4))
        waves = int(rng.integers(1, 40))
        ctx = rng.integers(0, 120, size=b)
        seen = {}
        for _, bb, h, unit, n in walk_entries(ctx, hkv, waves):
            for u in range(unit, unit + max(n, 1)):
                key = (bb, h, u)
                assert key not in seen
                seen[key] = 1
        want = sum(hkv * (c // 16 + (c % 16 > 0)) for c in ctx if c > 0)
        assert len(seen) == want
