"""An exact scalar re-derivation of the whole method on tiny tensors, against
the oracle (oracle.fp4).

Everything here is exact rational arithmetic (fractions.Fraction) with one
generic round-to-nearest-even routine for every finite binary format (binary32,
bf16, E4M3) written from the format definitions, so it shares nothing with the
oracle's NumPy float32 code: not its casts, tables or rounding helpers. Each
fp32(.) of the method is the exact rational result rounded once. It follows
the same readings as the oracle (module docstring of oracle/fp4.py) and checks
every output: block scales, global scales, codes, guidance planes, rollout and
guided outputs for bits 0..4, and Reconstruct.
"""

from fractions import Fraction as F

import numpy as np
import pytest

from oracle import formats, fp4

E2M1 = [F(0), F(1, 2), F(1), F(3, 2), F(2), F(3), F(4), F(6)]


def round_format(q: F, mbits: int, emin: int, maxval: F) -> F:
    """Round |q| to the nearest value of a binary format with mbits stored
    mantissa bits and smallest normal exponent emin (subnormals below), ties
    to even; results above maxval saturate to maxval (callers clamp first
    where the method says so)."""
    sign = -1 if q < 0 else 1
    q = abs(q)
    if q == 0:
        return F(0)
    e = emin
    if q >= F(2) ** emin:
        e = q.numerator.bit_length() - q.denominator.bit_length()
        while F(2) ** e > q:
            e -= 1
        while F(2) ** (e + 1) <= q:
            e += 1
    ulp = F(2) ** (e - mbits)
    k = q / ulp
    lo = k.numerator // k.denominator
    rem = k - lo
    if rem > F(1, 2) or (rem == F(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * ulp
    return sign * min(r, maxval)


F32_MAX = (2 - F(2) ** -23) * F(2) ** 127


def fp32(q: F) -> F:
    return round_format(q, 23, -126, F32_MAX) if abs(q) <= F32_MAX else (F32_MAX if q > 0 else -F32_MAX)


def bf16(q: F) -> F:
    return round_format(q, 7, -126, (2 - F(2) ** -7) * F(2) ** 127)


def e4m3(q: F) -> F:
    return round_format(q, 3, -6, F(448))


def from_bf16_bits(b: int) -> F:
    sign = -1 if b & 0x8000 else 1
    e, m = (b >> 7) & 0xFF, b & 0x7F
    if e == 0:
        return sign * F(m, 128) * F(2) ** -126
    return sign * (1 + F(m, 128)) * F(2) ** (e - 127)


def bits_of_bf16(v: F, negative: bool) -> int:
    """bf16 bit pattern of an exactly representable value with a sign bit."""
    a = abs(v)
    s = 0x8000 if negative else 0
    if a == 0:
        return s
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    if e < -126:
        return s | int(a / F(2) ** -133)
    m = (a / F(2) ** e - 1) * 128
    assert m.denominator == 1
    return s | ((e + 127) << 7) | int(m)


def rtn_index(t: F) -> int:
    if t > 6:
        return 7
    d = [abs(v - t) for v in E2M1]
    best = min(d)
    ks = [k for k in range(8) if d[k] == best]
    ev = [k for k in ks if k % 2 == 0]
    return ev[0] if ev else ks[0]


def bracket(t: F):
    if t >= 6:
        return 7, 7
    for k in range(8):
        if t == E2M1[k]:
            return k, k
    lo = max(k for k in range(8) if E2M1[k] < t)
    return lo, lo + 1


def reconstruct(t: F, c: int, b: int) -> int:
    best = None
    for k in range(8):
        if k % (1 << b) != c:
            continue
        d = abs(E2M1[k] - t)
        if best is None or d < best[0] or (d == best[0] and k > best[1]):
            best = (d, k)
    return best[1]


def choose(lo: int, hi: int, ref: F) -> int:
    return hi if abs(E2M1[hi] - ref) < abs(E2M1[lo] - ref) else lo


class Exact:
    """The method on one tensor, scalar and exact."""

    def __init__(self, fmt: int, bits_x, gscale=None):
        self.fmt = fmt
        self.B = 16 if fmt == fp4.NVFP4 else 32
        self.x = [from_bf16_bits(int(b)) for b in bits_x]
        self.neg = [bool(int(b) & 0x8000) for b in bits_x]
        if fmt == fp4.NVFP4:
            A = max((abs(v) for v in self.x), default=F(0))
            self.S = F(1) if A == 0 else fp32(F(2688) / A)
            if gscale is not None:
                self.S = gscale
            self.A = A

    def block_factors(self, blk):
        vals = self.x[blk * self.B:(blk + 1) * self.B]
        a = max(abs(v) for v in vals)
        if self.fmt == fp4.NVFP4:
            u = min(fp32(fp32(a / 6) * self.S), F(448))
            e = e4m3(u)
            if e == 0:
                return e, F(0), F(0)
            return e, fp32(e / self.S), min(fp32(self.S / e), F32_MAX)
        if a == 0:
            E = -127
        else:
            E = a.numerator.bit_length() - a.denominator.bit_length()
            while F(2) ** E > a:
                E -= 1
            while F(2) ** (E + 1) <= a:
                E += 1
            E = max(-127, min(127, E - 2))
        return E, F(2) ** E, F(2) ** -E

    def normalized(self, factors):
        """t and (d, scale id) per element under the given per-block factors."""
        out = []
        for i, v in enumerate(self.x):
            _, d, r = factors[i // self.B]
            out.append((fp32(abs(v) * r), d))
        return out

    def dequant(self, k, d, neg):
        return bits_of_bf16(bf16(fp32(E2M1[k] * d)), neg)


def _nblocks(n, B):
    return n // B


@pytest.mark.parametrize("fmt", [fp4.NVFP4, fp4.MXFP4])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_whole_method_exact_vs_oracle(fmt, seed):
    rng = np.random.default_rng(seed)
    n = 64
    # training and rollout tensors with a spread of magnitudes, zeros, ties
    xt = formats.f32_to_bf16((rng.standard_t(4, n) * np.exp(rng.normal(0, 1.5, n))).astype(np.float32))
    xt[::11] = 0
    xt[5::13] |= 0x8000
    xr = formats.f32_to_bf16((formats.bf16_to_f32(xt) * (1 + rng.normal(0, 0.05, n))).astype(np.float32))
    roll = Exact(fmt, xr)
    nb = _nblocks(n, roll.B)
    rf = [roll.block_factors(b) for b in range(nb)]
    tr = roll.normalized(rf)
    k_r = [rtn_index(t) for t, _ in tr]
    # the oracle
    for bits in (1, 2, 3, 4):
        o = fp4.encode_guidance(fmt, bits, xr)
        if fmt == fp4.NVFP4:
            assert F(float(o["gscale"])) == roll.S
            want_scales = [int(formats.e4m3_encode(np.array([float(e)], np.float32))[0]) for e, _, _ in rf]
        else:
            want_scales = [E + 127 for E, _, _ in rf]
        assert list(o["scales"]) == want_scales
        y_r = [roll.dequant(k_r[i], tr[i][1], roll.neg[i]) for i in range(n)]
        assert list(o["y"]) == y_r
        if bits < 4:
            assert list(fp4.unpack_low_bits(o["guide"], bits, n)) == [k & ((1 << bits) - 1) for k in k_r]
        else:
            assert list(fp4.unpack_codes(o["guide"])) == [(8 if roll.neg[i] else 0) | k_r[i] for i in range(n)]
        # training side under the rollout factors
        train = Exact(fmt, xt)
        tt = train.normalized(rf)
        for gb in (0, bits):
            og = fp4.guided_fake_quant(fmt, gb, xt, None if gb == 0 else o["guide"], o["scales"], o["gscale"])
            ks = []
            for i, (t, d) in enumerate(tt):
                if gb == 0:
                    k = rtn_index(t)
                else:
                    lo, hi = bracket(t)
                    if gb == 4:
                        same = train.neg[i] == roll.neg[i] or k_r[i] == 0
                        q_r = (-1 if roll.neg[i] else 1) * E2M1[k_r[i]]
                        s_t = -1 if train.neg[i] else 1
                        k = hi if abs(s_t * E2M1[hi] - q_r) < abs(s_t * E2M1[lo] - q_r) else lo
                        del same
                    else:
                        ref = reconstruct(t, k_r[i] & ((1 << gb) - 1), gb)
                        k = choose(lo, hi, E2M1[ref])
                ks.append(k)
            assert list(og["y"]) == [train.dequant(ks[i], tt[i][1], train.neg[i]) for i in range(n)], (bits, gb)
            assert list(fp4.unpack_codes(og["codes"])) == [(8 if train.neg[i] else 0) | ks[i] for i in range(n)]
        if bits < 4:
            ref_codes = fp4.unpack_codes(fp4.decode_guidance(fmt, xt, o["guide"], o["scales"], o["gscale"], bits))
            want = [(8 if train.neg[i] else 0) | reconstruct(tt[i][0], k_r[i] & ((1 << bits) - 1), bits)
                    for i in range(n)]
            assert list(ref_codes) == want


def test_exact_scale_corners_vs_oracle():
    """Tensors whose amax forces tiny and huge global scales, E4M3 subnormal
    and zero block scales, against the oracle."""
    cases = [
        [0x7F7F] + [0x0001] * 15 + [0x3F80] * 16,      # S clamps toward the smallest, zero blocks
        [0x0001] * 16 + [0x0002] * 16,                   # tiny amax: S clamps to FLT_MAX
        [0x4F00, 0x3000] + [0] * 14 + [0x2000] * 16,     # subnormal E4M3 block scales
    ]
    for xb in cases:
        xb = np.array(xb, np.uint16)
        ex = Exact(fp4.NVFP4, xb)
        o = fp4.quantize_rtn(fp4.NVFP4, xb)
        assert F(float(o["gscale"])) == ex.S
        rf = [ex.block_factors(b) for b in range(len(xb) // 16)]
        assert list(o["scales"]) == [int(formats.e4m3_encode(np.array([float(e)], np.float32))[0]) for e, _, _ in rf]
        tt = ex.normalized(rf)
        assert list(o["y"]) == [ex.dequant(rtn_index(t), d, ex.neg[i]) for i, (t, d) in enumerate(tt)]


def test_round_format_against_torch_casts():
    """The rounding routine itself against library casts (torch bf16 and
    float8_e4m3fn) on random and boundary values."""
    import torch
    rng = np.random.default_rng(4)
    vals = np.concatenate([rng.normal(0, 3, 500), 2.0 ** rng.uniform(-12, 8, 500),
                           [0.001953125, 0.0009765625, 0.00146484375, 448, 440, 464]]).astype(np.float32)
    for v in vals:
        fv = F(float(v))
        b = torch.tensor([float(v)], dtype=torch.float32).to(torch.bfloat16).to(torch.float32).item()
        assert bf16(fv) == F(b), v
        if abs(v) <= 448:
            e = torch.tensor([float(v)], dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float32).item()
            assert e4m3(fv) == F(e), v
