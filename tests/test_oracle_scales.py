"""Pins for the oracle's scaling and end-to-end calls: the paper's worked
examples (tests/golden/), closed forms, library casts, exhaustive bf16
enumeration in a block with unit scales, and MXFP4 exactness properties."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats, fp4

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

F32 = np.float32


def _bits(vals):
    return formats.f32_to_bf16(np.asarray(vals, dtype=np.float32))


def _f(bits):
    return formats.bf16_to_f32(bits).astype(np.float64)


def _example_pair(anchor, block_max, train, rollout):
    """Two 32-element tensors: block 0 holds the anchor (sets the tensor amax),
    block 1 holds [block_max, value, 0, ...]."""
    xt = np.zeros(32, np.float32)
    xt[0] = anchor
    xt[16] = block_max
    xr = xt.copy()
    xt[17] = train
    xr[17] = rollout
    return _bits(xt), _bits(xr)


def test_amplification_example(golden):
    g = golden("amplification_fig4a.json")
    p, d = g["printed"], g["derived"]
    bt, br = _example_pair(d["anchor_amax"], d["block_max"], p["train_value"], p["rollout_value"])
    assert _f(bt)[17] == d["train_bf16"] and _f(br)[17] == d["rollout_bf16"]
    assert abs((p["train_value"] - p["rollout_value"]) - p["bf16_difference"]) < 1e-9
    qt = fp4.quantize_rtn(fp4.NVFP4, bt)
    qr = fp4.quantize_rtn(fp4.NVFP4, br)
    assert qt["gscale"] == 1.0 and qt["amax"] == d["anchor_amax"]
    assert formats.e4m3_value(qt["scales"][1]) == d["block_scale"]
    assert np.array_equal(qt["scales"], qr["scales"])            # same global and block scales
    dd, r = fp4.nvfp4_block_factors(qt["scales"], qt["gscale"])
    tt = fp4.normalize(bt, r, 16)[17]
    tr = fp4.normalize(br, r, 16)[17]
    assert round(float(tt), 2) == p["normalized_train"]
    assert round(float(tr), 2) == p["normalized_rollout"]
    assert formats.E2M1[qt["k"][17]] == p["rtn_train"]
    assert formats.E2M1[qr["k"][17]] == p["rtn_rollout"]
    yt, yr = _f(qt["y"])[17], _f(qr["y"])[17]
    assert (yt, yr) == (d["train_dequant"], d["rollout_dequant"])
    assert abs(yt - yr) == p["fp4_discrepancy"]
    # guided, both record forms
    for bits in (1, 4):
        enc = fp4.encode_guidance(fp4.NVFP4, bits, br)
        gq = fp4.guided_fake_quant(fp4.NVFP4, bits, bt, enc["guide"], enc["scales"], enc["gscale"])
        assert abs(_f(gq["y"])[17] - yr) == d["guided_discrepancy"]
    # statistics over the tensor pair
    sb, sf, n = fp4.discrepancy_stats(bt, br, qt["y"], qr["y"])
    assert (sb, sf, n) == (d["sum_sq_bf16"], d["sum_sq_fp4_rtn"], 32.0)
    assert fp4.derived_metrics(sb, sf, n)["rel_excess"] == d["relative_excess_rtn"]
    enc = fp4.encode_guidance(fp4.NVFP4, 1, br)
    gq = fp4.guided_fake_quant(fp4.NVFP4, 1, bt, enc["guide"], enc["scales"], enc["gscale"])
    sb2, sf2, _ = fp4.discrepancy_stats(bt, br, gq["y"], enc["y"])
    assert fp4.derived_metrics(sb2, sf2, n)["rel_excess"] == d["relative_excess_guided"]


def test_example1_zero_discrepancy(golden):
    g = golden("example1_fig3.json")
    p, d = g["printed"], g["derived"]
    bt, br = _example_pair(d["anchor_amax"], d["block_max"], p["train_value"], p["rollout_value"])
    assert _f(bt)[17] == d["train_bf16"] and _f(br)[17] == d["rollout_bf16"]
    qt = fp4.quantize_rtn(fp4.NVFP4, bt)
    qr = fp4.quantize_rtn(fp4.NVFP4, br)
    assert formats.e4m3_value(qt["scales"][1]) == 1.0
    assert formats.E2M1[qt["k"][17]] == p["vanilla_fp4_train"]
    assert formats.E2M1[qr["k"][17]] == p["vanilla_fp4_rollout"]
    assert _f(qt["y"])[17] - _f(qr["y"])[17] == p["vanilla_discrepancy"]
    for bits in (0, 1, 4):
        enc = fp4.encode_guidance(fp4.NVFP4, 4 if bits == 0 else bits, br)
        gq = fp4.guided_fake_quant(fp4.NVFP4, bits, bt, enc["guide"], enc["scales"], enc["gscale"])
        assert _f(gq["y"])[17] - _f(enc["y"])[17] == p["guided_discrepancy"]


def test_global_scale_closed_form():
    assert fp4.nvfp4_global_scale(F32(2688.0)) == 1.0
    assert fp4.nvfp4_global_scale(F32(0.0)) == 1.0
    assert fp4.nvfp4_global_scale(F32(1e-38)) == formats.FLT_MAX
    rng = np.random.default_rng(5)
    for a in np.exp2(rng.uniform(-100, 100, 2000)).astype(np.float32):
        s = fp4.nvfp4_global_scale(a)
        exact = Fraction(2688) / Fraction(float(a))
        assert abs(Fraction(float(s)) - exact) <= exact * Fraction(1, 2 ** 24)


def test_tensor_amax_block_maps_to_top_scale():
    # The block holding the tensor amax gets E4M3 448 and its largest element
    # normalizes to (about) 6, the top codeword.
    rng = np.random.default_rng(1)
    for _ in range(50):
        x = _bits(rng.standard_t(4, 256).astype(np.float32) * np.exp(rng.normal()))
        q = fp4.quantize_rtn(fp4.NVFP4, x)
        a = np.abs(_f(x)).reshape(-1, 16).max(axis=1)
        top = int(np.argmax(a))
        assert formats.e4m3_value(q["scales"][top]) == 448.0
        i = int(np.argmax(np.abs(_f(x))))
        assert formats.E2M1[q["k"][i]] == 6.0


def test_nvfp4_block_scale_vs_torch_cast():
    # e is the E4M3 cast (torch, RNE) of min(fp32(fp32(a/6) * S), 448).
    rng = np.random.default_rng(2)
    x = _bits((rng.standard_t(4, 16 * 4000) * np.exp2(rng.uniform(-40, 40, 16 * 4000))).astype(np.float32))
    s = fp4.nvfp4_global_scale(fp4.tensor_amax(x))
    e = fp4.nvfp4_block_scales(x, s)
    a = np.abs(formats.bf16_to_f32(x)).reshape(-1, 16).max(axis=1)
    u = np.minimum((a / F32(6)).astype(F32) * s, F32(448)).astype(F32)
    ref = torch.from_numpy(u).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e, ref)
    assert np.any(e == 0) and np.any((e > 0) & (e < 8))      # zero and subnormal scales occur


def test_zero_scale_block_outputs_signed_zero():
    x = np.zeros(32, np.float32)
    x[0] = 1e30
    x[16:32] = np.linspace(-1e-20, 1e-20, 16)
    b = _bits(x)
    q = fp4.quantize_rtn(fp4.NVFP4, b)
    assert q["scales"][1] == 0
    assert np.all(q["k"][16:] == 0)
    assert np.array_equal(q["y"][16:], (b[16:] & 0x8000))
    assert np.array_equal(fp4.unpack_codes(q["codes"])[16:], ((b[16:] >> 15) << 3).astype(np.uint8))


def _brute_rtn_value(a):
    fa = Fraction(float(a))
    vs = [Fraction(v).limit_denominator() for v in formats.E2M1]
    if fa > 6:
        return 6.0
    d = [abs(v - fa) for v in vs]
    m = min(d)
    ks = [k for k in range(8) if d[k] == m]
    ks = [k for k in ks if k % 2 == 0] or ks
    return formats.E2M1[ks[0]]


def test_enumerate_all_bf16_members_under_unit_scales():
    """Every finite bf16 value with |x| <= 6 as a non-max member of a block
    whose max is 6, in a tensor whose amax is 2688: S = 1 and e = 1, so
    d = r = 1 and the output must be sign(x) * nearest-even E2M1 value of |x|.
    This reduces the whole NVFP4 pipeline to the textbook E2M1 rounding."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = formats.bf16_to_f32(bits)
    keep = np.isfinite(f) & (np.abs(f) <= 6.0)
    members = bits[keep]
    nb = len(members)
    per = 15
    nblk = -(-nb // per)
    x = np.zeros((nblk + 1, 16), np.uint16)
    x[0, 0] = _bits([2688.0])[0]
    x[1:, 0] = _bits([6.0])[0]
    flat = np.zeros(nblk * per, np.uint16)
    flat[:nb] = members
    x[1:, 1:] = flat.reshape(nblk, per)
    q = fp4.quantize_rtn(fp4.NVFP4, x.reshape(-1))
    assert q["gscale"] == 1.0
    assert np.all(formats.e4m3_value(q["scales"][1:]) == 1.0)
    y = formats.bf16_to_f32(q["y"]).reshape(nblk + 1, 16)[1:, 1:].reshape(-1)[:nb]
    ysign = (q["y"].reshape(nblk + 1, 16)[1:, 1:].reshape(-1)[:nb] >> 15)
    xs = formats.bf16_to_f32(members)
    table = {}
    for a in np.unique(np.abs(xs)):
        table[float(a)] = _brute_rtn_value(a)
    exp = np.array([table[float(abs(v))] for v in xs])
    assert np.array_equal(np.abs(y.astype(np.float64)), exp)
    assert np.array_equal(ysign, members >> 15)


def test_mxfp4_scale_closed_form_and_exact_dequant():
    rng = np.random.default_rng(4)
    x = _bits((rng.standard_t(4, 32 * 3000) * np.exp2(rng.uniform(-60, 60, 32 * 3000).repeat(1))).astype(np.float32))
    q = fp4.quantize_rtn(fp4.MXFP4, x)
    a = np.abs(formats.bf16_to_f32(x).astype(np.float64)).reshape(-1, 32).max(axis=1)
    e = q["scales"].astype(np.int64) - 127
    nz = a > 0
    # block max lands in [4, 8) after scaling by 2^-E
    assert np.all(a[nz] * np.exp2(-e[nz].astype(np.float64)) >= 4)
    assert np.all(a[nz] * np.exp2(-e[nz].astype(np.float64)) < 8)
    assert np.all(e[~nz] == -127)
    # dequantization is exact: y = +-v(k) * 2^E
    y = formats.bf16_to_f32(q["y"]).astype(np.float64)
    v = np.array(formats.E2M1)[q["k"]] * np.repeat(np.exp2(e.astype(np.float64)), 32)
    assert np.array_equal(np.abs(y), v)
    # idempotent: quantizing the output again changes nothing
    q2 = fp4.quantize_rtn(fp4.MXFP4, q["y"])
    assert np.array_equal(q2["y"], q["y"]) and np.array_equal(q2["scales"], q["scales"])


def test_mxfp4_tiny_and_zero_blocks():
    x = np.zeros(96, np.uint16)
    x[32] = 1                      # smallest bf16 subnormal, 2^-133
    x[64] = 0x8000                 # -0
    q = fp4.quantize_rtn(fp4.MXFP4, x)
    assert list(q["scales"]) == [0, 0, 0]          # E = -127 clamps
    # 2^-133 * 2^127 = 2^-6 -> rounds to 0 with sign +
    assert q["k"][32] == 0 and q["y"][64] == 0x8000


def test_mxfp4_rejects_global_scale():
    with pytest.raises(ValueError):
        fp4.quantize_rtn(fp4.MXFP4, np.zeros(32, np.uint16), gscale=1.0)


def test_stats_exact_small():
    rng = np.random.default_rng(9)
    for _ in range(20):
        n = 64
        xt = _bits(rng.normal(size=n).astype(np.float32))
        xr = _bits(rng.normal(size=n).astype(np.float32) * 3)
        yt = _bits(rng.normal(size=n).astype(np.float32))
        yr = _bits(rng.normal(size=n).astype(np.float32))
        sb, sf, cnt = fp4.discrepancy_stats(xt, xr, yt, yr)
        esb = sum((Fraction(float(a)) - Fraction(float(b))) ** 2 for a, b in zip(_f(xt), _f(xr)))
        esf = sum((Fraction(float(a)) - Fraction(float(b))) ** 2 for a, b in zip(_f(yt), _f(yr)))
        assert abs(Fraction(sb) - esb) <= esb * Fraction(1, 10 ** 12)
        assert abs(Fraction(sf) - esf) <= esf * Fraction(1, 10 ** 12)
        assert cnt == n


def test_derived_metrics_special_cases():
    m = fp4.derived_metrics(0.0, 0.0, 4.0)
    assert np.isnan(m["rel_excess"])
    assert fp4.derived_metrics(0.0, 1.0, 4.0)["rel_excess"] == float("inf")
    m = fp4.derived_metrics(2.0, 1.0, 4.0)
    assert m["rel_excess"] == -0.5 and m["D_BF16"] == 0.5 and m["D_FP4"] == 0.25
    assert m["D_act"] == 1.0
