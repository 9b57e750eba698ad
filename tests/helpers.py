"""Small test-side helpers: hand-built page tables over dense data.

These build tiny paged problems directly in the tests (independent of the
``workloads`` generator) so that oracle pins do not depend on it.
"""
from __future__ import annotations

import numpy as np


def to_f16_bits(x):
    return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def f16_values(x):
    """Round to fp16 and return the float64 values actually stored."""
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float64)


def paginate(dense_list, ps, Hkv, D, rng, pool_extra=3, fill_bits=0x7E00,
             dtype=np.uint16):
    """dense_list: per-request arrays [L_r, Hkv, D] of raw bits.  Returns
    (pool [P, ps, Hkv, D], indptr, indices, last_page_len) with pages placed
    by a random permutation, unused pages / tail slots set to ``fill_bits``."""
    n = [(len(d) + ps - 1) // ps for d in dense_list]
    used = sum(n)
    P = used + pool_extra
    perm = rng.permutation(P).astype(np.int32)
    pool = np.full((P, ps, Hkv, D), fill_bits, dtype)
    indptr = np.zeros(len(dense_list) + 1, np.int32)
    indices = []
    last = np.zeros(len(dense_list), np.int32)
    off = 0
    for r, d in enumerate(dense_list):
        pages = perm[off:off + n[r]]
        off += n[r]
        indices.extend(pages.tolist())
        indptr[r + 1] = indptr[r] + n[r]
        for t in range(len(d)):
            pool[pages[t // ps], t % ps] = d[t]
        last[r] = len(d) - (n[r] - 1) * ps if n[r] else 0
    return pool, indptr, np.asarray(indices, np.int32), last
