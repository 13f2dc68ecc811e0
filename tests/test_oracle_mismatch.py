"""Pins for the mismatch diagnostics of the oracle (§3.2 "Key Design",
Fig. 6): distances between training and rollout codes on the signed E2M1
grid, and the direction of guided corrections against RTN.

What pins them: a hand table of code pairs, an independent construction of
the grid distance from the ranks of the 15 distinct signed codeword values,
and invariants (histograms sum to n, symmetric, ±0 coincide)."""

import numpy as np

from oracle import formats, fp4


def _rank_distance(a, b):
    """|rank(value(a)) - rank(value(b))| among the 15 distinct signed values."""
    mags = np.array(formats.E2M1, dtype=np.float64)
    vals = np.unique(np.concatenate([-mags, mags]))          # -6 .. 6, one zero
    def val(c):
        c = np.asarray(c, dtype=np.int64)
        return np.where(c & 8, -mags[c & 7], mags[c & 7])
    ra = np.searchsorted(vals, val(a))
    rb = np.searchsorted(vals, val(b))
    return np.abs(ra - rb)


def test_hand_table():
    # (code_t, code_r, distance): ±0 coincide; 6 and -6 are 14 apart;
    # 2 (k=4) and 3 (k=5) adjacent; 0.5 and -0.5 two apart (0 between).
    table = [(0x0, 0x8, 0), (0x7, 0xF, 14), (0x4, 0x5, 1), (0x1, 0x9, 2),
             (0x3, 0x3, 0), (0xA, 0xB, 1), (0x6, 0x2, 4), (0x8, 0x1, 1)]
    for a, b, d in table:
        c = fp4.mismatch_counts(np.array([a]), np.array([b]), np.array([a]))
        assert c[d] == 1 and c[:15].sum() == 1, (a, b, d)


def test_distance_matches_rank_construction_on_all_pairs():
    a, b = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    a, b = a.reshape(-1), b.reshape(-1)
    d = np.abs(fp4.code_position(a) - fp4.code_position(b))
    assert np.array_equal(d, _rank_distance(a, b))


def test_histograms_and_directions():
    rng = np.random.default_rng(5)
    n = 10000
    t = rng.integers(0, 16, n)
    r = rng.integers(0, 16, n)
    bb = rng.integers(0, 16, n)
    c = fp4.mismatch_counts(t, r, bb)
    assert c.shape == (32,)
    assert c[:15].sum() == n and c[15:30].sum() == n
    assert np.array_equal(c[:15], np.bincount(_rank_distance(t, r), minlength=15))
    assert np.array_equal(c[15:30], np.bincount(_rank_distance(bb, r), minlength=15))
    # direction counts compare magnitudes only
    assert c[30] == np.count_nonzero((t & 7) > (bb & 7))
    assert c[31] == np.count_nonzero((t & 7) < (bb & 7))
    # swapping train and rollout leaves the first histogram unchanged
    assert np.array_equal(fp4.mismatch_counts(r, t, bb)[:15], c[:15])


def test_guided_never_farther_than_rtn_with_full_information():
    """§3.1 guarantee in grid terms: with the full rollout code, the guided
    code is never farther from it than RTN's, element by element."""
    rng = np.random.default_rng(6)
    t = rng.uniform(0, 7, 20000).astype(np.float32)
    s_t = rng.integers(0, 2, t.size).astype(np.uint8)
    k_r = rng.integers(0, 8, t.size).astype(np.uint8)
    s_r = rng.integers(0, 2, t.size).astype(np.uint8)
    lo, hi = fp4.bracket(t)
    kg = fp4.select_full(lo, hi, s_t, s_r, k_r)
    kb = fp4.rtn(t)
    cg, cb, cr = fp4.codes_of(s_t, kg), fp4.codes_of(s_t, kb), fp4.codes_of(s_r, k_r)
    dg = np.abs(fp4.code_position(cg) - fp4.code_position(cr))
    db = np.abs(fp4.code_position(cb) - fp4.code_position(cr))
    assert (dg <= db).all()
