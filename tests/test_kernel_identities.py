"""Arithmetic identities the HIP kernels rely on, checked on the CPU over
their whole input domain (the kernels themselves are checked against the
oracle on the GPU).

fp32(a / 6) for the NVFP4 block scale. The block scale formula divides the
block maximum a (a bf16 value) by 6 in binary32. The kernels compute it as one
binary64 product a * fl64(1/6), rounded once to binary32. The two agree for
every finite bf16 a: a has at most 8 significant bits, so a / 6 is never
close enough to a binary32 rounding boundary (nor to a tie) for the relative
error of fl64(1/6) (below 2^-53) to move it across one."""

import numpy as np


def _finite_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


def test_div6_equals_rounded_binary64_product_for_every_bf16():
    a = _finite_bf16_as_f32()
    assert a.size == 65280
    direct = a / np.float32(6.0)                                  # binary32 division, RNE
    via64 = (a.astype(np.float64) * (1.0 / 6.0)).astype(np.float32)
    assert np.array_equal(direct.view(np.uint32), via64.view(np.uint32))


def test_div6_identity_is_not_vacuous():
    """The same shortcut with a binary32 reciprocal (a * fl32(1/6)) does
    differ from the division somewhere, so the test above can fail."""
    a = _finite_bf16_as_f32()
    direct = a / np.float32(6.0)
    via32 = a * np.float32(1.0 / 6.0)
    assert np.count_nonzero(direct.view(np.uint32) != via32.view(np.uint32)) > 0
