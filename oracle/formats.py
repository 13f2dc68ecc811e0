"""Number formats: bf16, FP4 E2M1, FP8 E4M3 (OCP "fn" variant) and E8M0.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The paper quantizes to FP4 E2M1 codewords with block scales (TRACE §3.1,
"Key Design", Fig. 4(a)); NVFP4 carries an E4M3 scale per 16 elements and an
FP32 global scale, MXFP4 an E8M0 power-of-two scale per 32 elements (§4.3,
"Performance Under Microscaling FP4 Formats"). The encodings below are the
textbook definitions of those formats; the paper only names them.
"""

from __future__ import annotations

import numpy as np

# E2M1 magnitudes by 3-bit index k = (exponent << 1) | mantissa, exponent bias 1,
# exponent 0 subnormal. The mantissa bit of index k is k & 1.
E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
E2M1_F32 = np.array(E2M1, dtype=np.float32)
E2M1_MAX = 6.0

FLT_MAX = np.float32(np.finfo(np.float32).max)


# --------------------------------------------------------------------------- bf16

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact: bf16 is the top
    half of a binary32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    The 16 discarded bits are compared with the halfway pattern 0x8000; a tie
    rounds so that the kept low bit is 0. Inputs must be finite (a carry out of
    the largest finite binade would give Inf, as IEEE rounding does).
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = b >> 16
    rest = b & 0xFFFF
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & 1) == 1))
    return (keep + up.astype(np.uint64)).astype(np.uint16)


# --------------------------------------------------------------------------- E4M3

def e4m3_value(byte: np.ndarray) -> np.ndarray:
    """Decode OCP FP8 E4M3 ("fn": bias 7, no infinities, S.1111.111 is NaN).

    Exponent field 0 is subnormal: value = (m / 8) * 2^-6. Otherwise
    value = (1 + m / 8) * 2^(E - 7). Returned as float32 (every E4M3 value is
    exactly representable there).
    """
    byte = np.asarray(byte, dtype=np.uint8).astype(np.int64)
    sign = np.where(byte & 0x80, -1.0, 1.0)
    exp = (byte >> 3) & 0xF
    man = byte & 0x7
    mag = np.where(exp == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(exp - 7.0))
    val = sign * mag
    val = np.where((byte & 0x7F) == 0x7F, np.nan, val)
    return val.astype(np.float32)


# All non-negative finite E4M3 values in ascending order; index == byte.
_E4M3_POS = e4m3_value(np.arange(0x7F, dtype=np.uint8)).astype(np.float64)
E4M3_MAX = float(_E4M3_POS[-1])   # 448


def e4m3_encode(u: np.ndarray) -> np.ndarray:
    """Nearest non-negative E4M3 value to u, ties to the even byte (mantissa
    LSB 0); u must lie in [0, 448]. This is IEEE round-to-nearest-even onto
    the E4M3 value set, subnormals included: anything at or below 2^-10 (half
    the smallest subnormal 2^-9) becomes 0.
    """
    u = np.asarray(u, dtype=np.float32).astype(np.float64)
    if np.any(~(u >= 0)) or np.any(u > E4M3_MAX):
        raise ValueError("e4m3_encode expects values in [0, 448]")
    hi = np.searchsorted(_E4M3_POS, u, side="left")      # first value >= u
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = u - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - u
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    out = np.where(pick_hi, hi, lo)
    out = np.where(_E4M3_POS[hi] == u, hi, out)          # exact hits
    return out.astype(np.uint8)


# --------------------------------------------------------------------------- E8M0

def floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for positive finite a, exactly, from the binary exponent
    (frexp gives a = m * 2^e with m in [0.5, 1), so floor(log2 a) = e - 1)."""
    _, e = np.frexp(np.asarray(a, dtype=np.float64))
    return e.astype(np.int64) - 1

