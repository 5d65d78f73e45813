"""The host replica of the decode stream's work split (tests/unit_split.py),
which the GPU tests use to know which kernel route a case exercises, checked
against a unit-by-unit walk of the same rules on random small cases; and the
identity the split merge's slot walk rests on."""

import numpy as np
import pytest

from tests.unit_split import completion_kinds, units_of, walk_entries


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


@pytest.mark.parametrize("case", range(30))
def test_merge_slot_walk_matches_owner_span(case):
    """The merge's slot walk: with fewer units than waves (U < W) every
    non-empty range holds exactly one unit, so the waves with non-empty ranges
    between a (sequence, head)'s first and last owner are exactly the owners of
    its units, and the first owner's range starts at the pair's first unit;
    with U >= W no range is empty."""
    rng = np.random.default_rng(500 + case)
    b = int(rng.integers(1, 12))
    hkv = int(rng.choice([1, 2, 8]))
    ctx = rng.integers(0, 300, size=b)
    waves = int(rng.choice([64, 512, 2048]))
    units = units_of(ctx)
    U = int(hkv * units.sum())
    if U == 0:
        return
    owner = lambda u: ((u + 1) * waves - 1) // U
    nonempty = lambda w: w * U // waves < (w + 1) * U // waves
    if U >= waves:
        assert all(nonempty(w) for w in range(waves))
    first = 0
    for bb in range(b):
        for _ in range(hkv):
            n = int(units[bb])
            if n:
                x, y = owner(first), owner(first + n - 1)
                span = [w for w in range(x, y + 1) if nonempty(w)]
                if U < waves:
                    assert x * U // waves == first
                    assert span == [owner(first + k) for k in range(n)]
                else:
                    assert span == list(range(x, y + 1))
            first += n
