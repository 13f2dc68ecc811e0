"""Pins for oracle.record.gather_pages: a hand example, a byte-by-byte loop
on small pools, and the invariants of a page gather (an identity list returns
the pool, a permutation followed by its inverse returns the input, bad ids
give zero pages and are counted)."""

import numpy as np
import pytest

from oracle import record


def test_hand_example():
    pool = np.arange(12, dtype=np.uint8)               # 4 pages of 3 bytes
    out, bad = record.gather_pages(pool, 3, [2, 0, 7, 2, -1])
    assert list(out) == [6, 7, 8, 0, 1, 2, 0, 0, 0, 6, 7, 8, 0, 0, 0]
    assert bad == 2


@pytest.mark.parametrize("page_bytes", [1, 5, 16, 48])
def test_bytewise_loop(page_bytes):
    rng = np.random.default_rng(page_bytes)
    npool = 9
    pool = rng.integers(0, 256, npool * page_bytes).astype(np.uint8)
    ids = rng.integers(-2, npool + 2, 40)
    out, bad = record.gather_pages(pool, page_bytes, ids)
    want = []
    for i in ids:
        for b in range(page_bytes):
            want.append(int(pool[i * page_bytes + b]) if 0 <= i < npool else 0)
    assert list(out) == want
    assert bad == sum(1 for i in ids if not 0 <= i < npool)


def test_identity_and_inverse_permutation():
    rng = np.random.default_rng(1)
    pool = rng.integers(0, 256, 32 * 24).astype(np.uint8)
    out, bad = record.gather_pages(pool, 24, np.arange(32))
    assert bad == 0 and np.array_equal(out, pool)
    perm = rng.permutation(32)
    fwd, _ = record.gather_pages(pool, 24, perm)
    back, _ = record.gather_pages(fwd, 24, np.argsort(perm))
    assert np.array_equal(back, pool)


def test_rejects_partial_pages():
    with pytest.raises(ValueError):
        record.gather_pages(np.zeros(10, np.uint8), 3, [0])
