"""Comparison rules between the GPU path and the CPU oracle.

* int4 codes and fp16 scale/zero bit patterns: bit-exact, compared in logical
  (token, channel) order after decoding the GPU page bytes with tests/layout.py.
* tails: bit-exact fp16.
* attention output: max |O_gpu - O_ref| <= 2e-3 and
  ||O_gpu - O_ref||_2 / ||O_ref||_2 <= 1e-3 over all checked outputs of a case.
"""

import numpy as np

from tests import layout

TOL_MAX_ABS = 2e-3
TOL_REL_L2 = 1e-3


def page_mismatches(gpu_raw, oracle_pages, bits=4):
    """Compare GPU chunks (uint8 [n, Hkv, STRIDE]) with oracle pages
    (flush_pages output with leading dims [n, Hkv]). Returns a list of
    (field, count) for fields that differ; empty when bit-exact. bits=2 reads
    the 2-bit page format."""
    got = layout.read_chunks(gpu_raw) if bits == 4 else layout.read_chunks2(gpu_raw)
    bad = []
    for key in ("ck", "cv"):
        n = int(np.count_nonzero(got[key] != oracle_pages[key]))
        if n:
            bad.append((key, n))
    for key in ("sk", "zk", "sv", "zv"):
        want = np.ascontiguousarray(oracle_pages[key]).view(np.uint16)
        n = int(np.count_nonzero(got[key] != want))
        if n:
            bad.append((key, n))
    return bad


def attention_errors(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    diff = got - want
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.linalg.norm(want))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def attention_ok(got, want):
    max_abs, rel = attention_errors(got, want)
    return max_abs <= TOL_MAX_ABS and rel <= TOL_REL_L2, max_abs, rel
