"""Pins for oracle.formats: bf16 and E4M3 against torch's CPU casts (library
routines independent of the oracle), floor(log2) against exact comparisons."""

import math

import numpy as np
import pytest
import torch

from oracle import formats

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _finite_f32_patterns(n, seed):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    x = b.view(np.float32)
    return x[np.isfinite(x)]


def test_bf16_roundtrip_exact():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = formats.bf16_to_f32(bits)
    ok = np.isfinite(f)
    assert np.array_equal(formats.f32_to_bf16(f[ok]), bits[ok])
    # and bf16_to_f32 agrees with torch's widening
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(f.view(np.uint32)[ok], t.view(np.uint32)[ok])


@pytest.mark.parametrize("seed", [0, 1])
def test_f32_to_bf16_matches_torch_random(seed):
    x = _finite_f32_patterns(400_000, seed)
    x = x[np.abs(x) < 3.38e38]      # stay clear of rounding into Inf
    ours = formats.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f32_to_bf16_ties_and_subnormals():
    base = np.arange(0, 65536, 37, dtype=np.uint32) << 16
    cand = []
    for off in (0x7FFF, 0x8000, 0x8001, 0x0001, 0xFFFF):
        cand.append(base | off)
    cand.append(np.arange(0, 1 << 20, 3, dtype=np.uint32))  # fp32 subnormals
    b = np.concatenate(cand).astype(np.uint32)
    x = b.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.38e38)]
    ours = formats.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ours = formats.e4m3_value(b)
    ref = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert formats.E4M3_MAX == 448.0


def _e4m3_torch(u):
    return torch.from_numpy(np.asarray(u, dtype=np.float32).copy()).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_dense():
    vals = formats.e4m3_value(np.arange(0x7F, dtype=np.uint8)).astype(np.float32)
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    pts = [vals, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))]
    rng = np.random.default_rng(3)
    pts.append(np.exp2(rng.uniform(-14, np.log2(448), 300_000)).astype(np.float32))
    pts.append(rng.uniform(0, 448, 300_000).astype(np.float32))
    pts.append(np.array([0.0, 2 ** -10, 1.5 * 2 ** -10, 2 ** -9, 2 ** -11, 1e-30, 448.0,
                         447.9, 2 ** -149], dtype=np.float32))
    u = np.concatenate(pts)
    u = u[(u >= 0) & (u <= 448)]
    assert np.array_equal(formats.e4m3_encode(u), _e4m3_torch(u))


def test_e4m3_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        formats.e4m3_encode(np.array([449.0], dtype=np.float32))


def test_floor_log2_exact_all_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)   # positive finite
    a = formats.bf16_to_f32(bits).astype(np.float64)
    fl = formats.floor_log2(a)
    lo = np.ldexp(1.0, fl)
    hi = np.ldexp(1.0, fl + 1)
    assert np.all(lo <= a) and np.all(a < hi)
    for v in (1.0, 1.5, 2.0, 3.999, 4.0, 2.0 ** -133, 3.0e38):
        assert formats.floor_log2(np.array([v]))[0] == math.frexp(v)[1] - 1


def test_e2m1_table_is_textbook():
    # E2M1, bias 1: exponent 0 subnormal (0, 0.5); otherwise (1 + m/2) * 2^(e-1).
    vals = []
    for k in range(8):
        e, m = k >> 1, k & 1
        vals.append(m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))
    assert tuple(vals) == formats.E2M1
