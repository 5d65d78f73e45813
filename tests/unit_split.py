"""Host replica of the decode stream's work split (test infrastructure).

The int4 decode stream lays its units out sequence-major, then KV head, then
page, a unit being one full page or a non-empty fp16 tail; wave w of a grid of
W waves takes units [w U / W, (w + 1) U / W). Inside its range a wave pairs
consecutive full pages of one (sequence, head), starting from the first unit
of that (sequence, head) in its range; a page left over at the end of a range
or of a (sequence, head) is a single entry. The tests use this to find out
which route through the kernel a case takes.
"""

import numpy as np


def units_of(ctx):
    ctx = np.asarray(ctx, dtype=np.int64)
    return np.where(ctx > 0, ctx // 16 + (ctx % 16 > 0), 0)


def completion_kinds(ctx_after, hkv, waves):
    """How each page completed by a decode step's new token enters the stream.

    ``ctx_after``: context lengths counting the new token; a sequence whose
    length is a positive multiple of 16 has just completed its last page, the
    last unit of each of its (sequence, head) pairs. Returns (pair_b, single):
    how many of those pages are consumed as page B of a pair, and how many as
    a single page. Closed form of :func:`walk_entries`."""
    ctx = np.asarray(ctx_after, dtype=np.int64)
    units = units_of(ctx)
    U = int(hkv * units.sum())
    start = hkv * (np.cumsum(units) - units)
    pair_b = single = 0
    for b in np.nonzero((ctx > 0) & (ctx % 16 == 0))[0]:
        for h in range(hkv):
            seg0 = int(start[b]) + h * int(units[b])
            last = int(units[b]) - 1
            u = seg0 + last
            w = ((u + 1) * waves - 1) // U
            first_in_range = max(0, w * U // waves - seg0)
            if (last - first_in_range) % 2:
                pair_b += 1
            else:
                single += 1
    return pair_b, single


def walk_entries(ctx, hkv, waves):
    """Entries of every wave, walked unit by unit as the stream's cursors do:
    a list of (wave, b, h, first_unit, n_pages) for page entries (n_pages 1 or
    2) and n_pages 0 for a tail. Slow; for small cases."""
    ctx = np.asarray(ctx, dtype=np.int64)
    units = units_of(ctx)
    flat = []
    for b in range(len(ctx)):
        full = int(ctx[b]) // 16 if ctx[b] > 0 else 0
        for h in range(hkv):
            for u in range(int(units[b])):
                flat.append((b, h, u, full))
    U = len(flat)
    out = []
    for w in range(waves):
        u0, u1 = w * U // waves, (w + 1) * U // waves
        u = u0
        while u < u1:
            b, h, unit, full = flat[u]
            if unit >= full:
                out.append((w, b, h, unit, 0))
                u += 1
                continue
            n = 2 if (unit + 1 < full and u + 1 < u1) else 1
            out.append((w, b, h, unit, n))
            u += n
    return out
