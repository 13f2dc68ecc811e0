"""The record path around the guided kernels: how a finished request's
guidance is collected before it leaves the GPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

§3.2 "Motivation" and "Key Design" of the paper: records are kept per
trajectory, token and site during generation and moved to the training side
afterwards; for KV guidance the codes already sit in the FP4 KV cache. A paged
cache holds a request's tokens in fixed-size pages scattered over a pool, so
at request end its pages are gathered into one contiguous record before the
device-to-host copy. The pages say nothing about the layout; the reading here
is the plainest one: out[i] = pool[page_ids[i]], whole pages of page_bytes
bytes, and an id outside the pool yields a page of zero bytes (counted), so a
bad id can never read outside the pool.
"""

from __future__ import annotations

import numpy as np


def gather_pages(pool, page_bytes: int, page_ids):
    """(out uint8[n * page_bytes], bad_ids) with out's page i = pool page
    page_ids[i] (pool: uint8[pool_pages * page_bytes])."""
    pool = np.asarray(pool, dtype=np.uint8).reshape(-1)
    if page_bytes <= 0 or pool.size % page_bytes:
        raise ValueError("pool must hold whole pages")
    pages = pool.reshape(-1, page_bytes)
    ids = np.asarray(page_ids, dtype=np.int64).reshape(-1)
    ok = (ids >= 0) & (ids < pages.shape[0])
    out = np.zeros((ids.size, page_bytes), dtype=np.uint8)
    out[ok] = pages[ids[ok]]
    return out.reshape(-1), int(np.count_nonzero(~ok))
