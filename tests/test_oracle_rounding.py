"""Pins for the E2M1 rounding steps of the oracle: RTN, BracketFP4,
Reconstruct and the two selection rules.

What pins them: the paper's worked values (2.51 -> 3, 2.49 -> 2), brute force
with exact rationals, invariants (bracket contains t; the local guarantee of
§3.1), and hand-derived tables in tests/golden/.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats, fp4

V = [Fraction(v).limit_denominator() for v in formats.E2M1]


def _t_grid():
    """Every E2M1 magnitude, every midpoint, each +-1 ulp, plus random t."""
    pts = []
    vals = np.array(formats.E2M1, dtype=np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    for p in np.concatenate([vals, mids, [7.0, 8.0, 100.0]]).astype(np.float32):
        pts += [p, np.nextafter(p, np.float32(0)), np.nextafter(p, np.float32(1e9))]
    rng = np.random.default_rng(11)
    pts = np.array(pts, dtype=np.float32)
    return np.concatenate([pts, rng.uniform(0, 7, 20000).astype(np.float32),
                           np.float32(2.0) ** rng.uniform(-30, 3, 2000).astype(np.float32)])


def _brute_rtn(t):
    """Nearest E2M1 magnitude by exact distance; ties to the even index;
    saturate at 6."""
    ft = Fraction(float(t))
    if ft > 6:
        return 7
    d = [abs(v - ft) for v in V]
    m = min(d)
    ks = [k for k in range(8) if d[k] == m]
    even = [k for k in ks if k % 2 == 0]
    return even[0] if even else ks[0]


def test_rtn_printed_values():
    # §3.1, Fig. 4(a): normalized 2.51 rounds to 3, 2.49 to 2.
    k = fp4.rtn(np.array([2.51, 2.49], dtype=np.float32))
    assert [formats.E2M1[i] for i in k] == [3.0, 2.0]


def test_rtn_bruteforce():
    t = _t_grid()
    k = fp4.rtn(t)
    exp = np.array([_brute_rtn(x) for x in t], dtype=np.uint8)
    assert np.array_equal(k, exp)


def test_rtn_ties_go_to_mantissa_zero():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    k = fp4.rtn(mids)
    assert np.all(k % 2 == 0)
    assert [formats.E2M1[i] for i in k] == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]


def test_bracket_invariants():
    t = _t_grid()
    lo, hi = fp4.bracket(t)
    v = np.array(formats.E2M1)
    sat = t >= 6
    assert np.all(lo[sat] == 7) and np.all(hi[sat] == 7)
    ns = ~sat
    assert np.all(v[lo[ns]] <= t[ns]) and np.all(t[ns] <= v[hi[ns]])
    assert np.all((hi.astype(int) - lo.astype(int)) >= 0)
    assert np.all((hi.astype(int) - lo.astype(int)) <= 1)
    is_code = np.isin(t, np.array(formats.E2M1, dtype=np.float32))
    assert np.array_equal(lo[ns] == hi[ns], is_code[ns])
    # strictly inside the bracket when the candidates differ
    two = lo != hi
    assert np.all(v[lo[two]] < t[two]) and np.all(t[two] < v[hi[two]])
    # RTN always picks one of the two candidates (same candidate set, §3.1)
    k = fp4.rtn(t)
    assert np.all((k == lo) | (k == hi))


def _brute_reconstruct(t, c, b=1):
    ft = Fraction(float(t))
    best = None
    for k in range(8):
        if k % (2 ** b) != c:
            continue
        d = abs(V[k] - ft)
        if best is None or d < best[0] or (d == best[0] and k > best[1]):
            best = (d, k)
    return best[1]


def test_reconstruct_bruteforce():
    t = _t_grid()[:6000]
    for c in (0, 1):
        r = fp4.reconstruct(t, np.full(t.shape, c))
        exp = np.array([_brute_reconstruct(x, c) for x in t])
        assert np.array_equal(r, exp)
        assert np.all((r & 1) == c)


@pytest.mark.parametrize("b", [2, 3])
def test_reconstruct_low_b_bits_bruteforce(b):
    """Algorithm 1 prose with b = 2 and 3: nearest magnitude whose low b index
    bits equal c, exact rationals, ties to the larger magnitude."""
    t = _t_grid()[:3000]
    for c in range(2 ** b):
        r = fp4.reconstruct(t, np.full(t.shape, c), b)
        exp = np.array([_brute_reconstruct(x, c, b) for x in t])
        assert np.array_equal(r, exp)
        assert np.all((r & (2 ** b - 1)) == c)


def test_reconstruct_b3_is_the_rollout_magnitude():
    """b = 3 keeps the whole magnitude index: one candidate, whatever t is."""
    t = _t_grid()
    for c in range(8):
        assert np.all(fp4.reconstruct(t, np.full(t.shape, c), 3) == c)


def test_reconstruct_b2_thresholds():
    """b = 2 chooses between index c and c + 4 (magnitudes {0, 2}, {.5, 3},
    {1, 4}, {1.5, 6}); the upper one from the midpoint 1, 1.75, 2.5, 3.75 on
    (inclusive: ties go up). Derived by hand from the E2M1 table."""
    mid = {0: 1.0, 1: 1.75, 2: 2.5, 3: 3.75}
    for c, m in mid.items():
        m32 = np.float32(m)
        t = np.array([0, np.nextafter(m32, np.float32(0)), m32, np.nextafter(m32, np.float32(9)), 7],
                     dtype=np.float32)
        assert list(fp4.reconstruct(t, np.full(5, c), 2)) == [c, c, c + 4, c + 4, c + 4]


@pytest.mark.parametrize("b", [1, 2, 3])
def test_low_bit_guidance_adjacent_guarantee(b):
    """For every b: where the rollout magnitude is a candidate, the guided
    index is the rollout's or RTN's (local guarantee); with b = 3 it is always
    the rollout's there, and b = 3 equals the full-code selection when the
    signs agree."""
    t = _t_grid()
    t = t[t < 6]
    lo, hi = fp4.bracket(t)
    k_rtn = fp4.rtn(t)
    zeros = np.zeros(t.shape, np.uint8)
    v = np.array(formats.E2M1)
    for k_r in range(8):
        kr = np.full(t.shape, k_r, np.uint8)
        kg = fp4.select_compact(lo, hi, fp4.reconstruct(t, kr & (2 ** b - 1), b))
        assert np.all((kg == lo) | (kg == hi))
        adj = (kr == lo) | (kr == hi)
        assert np.all((kg[adj] == kr[adj]) | (kg[adj] == k_rtn[adj]))
        assert np.all(np.abs(v[kg[adj]] - v[k_r]) <= np.abs(v[k_rtn[adj]] - v[k_r]))
        if b == 3:
            assert np.all(kg[adj] == kr[adj])
            assert np.array_equal(kg, fp4.select_full(lo, hi, zeros, zeros, kr))


def test_compact_select_table(golden):
    g = golden("compact_select_table.json")
    rows = np.array(g["rows"], dtype=np.float64)
    t = rows[:, 0].astype(np.float32)
    c = rows[:, 1].astype(np.int64)
    r = fp4.reconstruct(t, c)
    lo, hi = fp4.bracket(t)
    k = fp4.select_compact(lo, hi, r)
    v = np.array(formats.E2M1)
    assert np.array_equal(v[r], rows[:, 2])
    assert np.array_equal(v[k], rows[:, 3])


def test_full_select_table(golden):
    g = golden("full_select_table.json")
    rows = np.array(g["rows"], dtype=np.float64)
    t = rows[:, 0].astype(np.float32)
    q = rows[:, 1]
    s_r = (np.signbit(q)).astype(np.uint8)
    k_r = np.array([formats.E2M1.index(abs(x)) for x in q], dtype=np.uint8)
    lo, hi = fp4.bracket(t)
    k = fp4.select_full(lo, hi, np.zeros(t.shape, np.uint8), s_r, k_r)
    v = np.array(formats.E2M1)
    assert np.array_equal(v[k], rows[:, 2])
    assert np.array_equal(v[fp4.rtn(t)], rows[:, 3])


def _all_signed_codes():
    return [(s, k) for s in (0, 1) for k in range(8)]


def test_full_information_guarantee_exhaustive():
    """§3.1: |q_TRACE - q_rollout| <= |q_RTN - q_rollout| for every element,
    under the same scale and candidate set."""
    t = _t_grid()
    lo, hi = fp4.bracket(t)
    k_rtn = fp4.rtn(t)
    for s_t in (0, 1):
        st = np.full(t.shape, s_t, np.uint8)
        for s_r, k_r in _all_signed_codes():
            sr = np.full(t.shape, s_r, np.uint8)
            kr = np.full(t.shape, k_r, np.uint8)
            kg = fp4.select_full(lo, hi, st, sr, kr)
            q_r = fp4.signed_value(sr, kr)
            dg = np.abs(fp4.signed_value(st, kg) - q_r)
            dn = np.abs(fp4.signed_value(st, k_rtn) - q_r)
            assert np.all(dg <= dn)
            assert np.all((kg == lo) | (kg == hi))
            # A rollout codeword inside the candidate set with the training
            # sign is reproduced exactly (zero local discrepancy).
            inside = ((kr == lo) | (kr == hi)) & ((sr == st) | (kr == 0))
            assert np.all(kg[inside] == kr[inside])


def test_compact_conditional_guarantee():
    """b = 1: where the rollout magnitude is one of the two candidates and the
    signs agree, the guided index is either the rollout's or RTN's, so the
    local guarantee holds there; it is the rollout's whenever the
    reconstructed reference is itself a candidate."""
    t = _t_grid()
    t = t[t < 6]
    lo, hi = fp4.bracket(t)
    k_rtn = fp4.rtn(t)
    for k_r in range(8):
        kr = np.full(t.shape, k_r, np.uint8)
        c = kr & 1
        r = fp4.reconstruct(t, c)
        kg = fp4.select_compact(lo, hi, r)
        assert np.all((kg == lo) | (kg == hi))
        adj = (kr == lo) | (kr == hi)
        assert np.all((kg[adj] == kr[adj]) | (kg[adj] == k_rtn[adj]))
        v = np.array(formats.E2M1)
        assert np.all(np.abs(v[kg[adj]] - v[k_r]) <= np.abs(v[k_rtn[adj]] - v[k_r]))
        ref_in = adj & ((r == lo) | (r == hi))
        assert np.all(kg[ref_in] == kr[ref_in])


def test_compact_can_lose_outside_the_adjacent_case():
    # Not a guarantee beyond adjacency (Algorithm 1 prose: the reference is a
    # guidance target, not an exact recovery): t = 2.6, rollout 4 (c = 0)
    # reconstructs 2 and picks 2, while RTN picks 3, closer to 4.
    t = np.array([2.6], dtype=np.float32)
    lo, hi = fp4.bracket(t)
    r = fp4.reconstruct(t, np.array([0]))
    assert formats.E2M1[fp4.select_compact(lo, hi, r)[0]] == 2.0
    assert formats.E2M1[fp4.rtn(t)[0]] == 3.0


def test_pack_layouts():
    codes = np.array([0x1, 0x2, 0xF, 0x8, 0x7, 0x0], dtype=np.uint8)
    assert list(fp4.pack_codes(codes)) == [0x21, 0x8F, 0x07]
    assert np.array_equal(fp4.unpack_codes(fp4.pack_codes(codes)), codes)
    bits = np.array([1, 0, 0, 0, 0, 0, 0, 1, 0, 1, 0, 0, 0, 0, 0, 0], dtype=np.uint8)
    assert list(fp4.pack_bits(bits)) == [0x81, 0x02]
    assert np.array_equal(fp4.unpack_bits(fp4.pack_bits(bits)), bits)
    # b = 1 is pack_bits
    assert np.array_equal(fp4.pack_low_bits(bits, 1), fp4.pack_bits(bits))
    # b = 2: element 4j + i at bits 2i of byte j
    two = np.array([1, 2, 3, 0, 0, 0, 0, 3], dtype=np.uint8)
    assert list(fp4.pack_low_bits(two, 2)) == [0b00111001, 0b11000000]
    # b = 3: element 8j + i at bits 3i of the 24-bit little-endian group j
    three = np.array([7, 0, 5, 1, 2, 3, 4, 6], dtype=np.uint8)
    word = sum(int(x) << (3 * i) for i, x in enumerate(three))
    assert list(fp4.pack_low_bits(three, 3)) == [word & 0xFF, (word >> 8) & 0xFF, word >> 16]
    rng = np.random.default_rng(3)
    for b in (1, 2, 3):
        vals = rng.integers(0, 2 ** b, 64).astype(np.uint8)
        packed = fp4.pack_low_bits(vals, b)
        assert packed.size == fp4.guide_bytes(b, 64) == 8 * b
        assert np.array_equal(fp4.unpack_low_bits(packed, b, 64), vals)
