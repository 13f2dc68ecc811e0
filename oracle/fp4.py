"""The method: block-scaled FP4 fake quantization, rollout guidance and
rollout-guided rounding, step by step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Citations name sections of "TRACE: Rollout-Guided Quantization-Aware Training
for FP4 Reinforcement Learning of MoE Language Models" (reader view).

Arrays are flat: an input tensor [rows, cols] with cols a multiple of the block
size B is a sequence of N / B blocks of B consecutive elements. Inputs are bf16
bit patterns (uint16). Per-element results (indices, codes) are unpacked here;
``pack_codes`` / ``pack_bits`` give the byte planes the library writes.

Readings where the paper is silent (each is listed, with its reason, in the
design notes of the repository):

* NVFP4 scales. A = max|x| over the tensor; S = 2688 / A (2688 = 6 * 448, so
  the largest block maps onto the top E4M3 scale), 1 when A = 0, clamped to
  FLT_MAX. Per block: u = fp32(fp32(a / 6) * S), e = E4M3_RNE(min(u, 448)),
  d = fp32(e / S) (decode factor), r = min(fp32(S / e), FLT_MAX) (encode
  factor); a zero scale byte gives d = r = 0. The normalized value is
  t = fp32(|x| * r). All binary32, no fused multiply-add.
* MXFP4 scale. E = clamp(floor(log2 a) - 2, -127, 127), -127 for an all-zero
  block; the byte is E + 127; t = fp32(|x| * 2^-E), d = 2^E.
* RTN rounds t to the nearest E2M1 magnitude, ties to the even index
  (mantissa 0), and saturates above 6.
* Signs: every code and output carries the sign bit of its own input, so a
  negative value that rounds to 0 gives code 0x8 and bf16 -0.0.
* Bracket, at an exact codeword or at t >= 6, is the single codeword.
* Reconstruct breaks its (rare) ties toward the larger magnitude.
* The training side always uses the rollout's scales.
"""

from __future__ import annotations

import numpy as np

from .formats import (E2M1_F32, FLT_MAX, bf16_to_f32, e4m3_encode, e4m3_value,
                      f32_to_bf16, floor_log2)

NVFP4, MXFP4 = 0, 1
BLOCK = {NVFP4: 16, MXFP4: 32}
NVFP4_GLOBAL_NUM = np.float32(6.0 * 448.0)   # 2688
_F32 = np.float32


def _u16(x):
    return np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)


def _sign(x_bits):
    return (np.asarray(x_bits, dtype=np.uint16) >> 15).astype(np.uint8)


def _abs_f32(x_bits):
    return bf16_to_f32(np.asarray(x_bits, dtype=np.uint16) & 0x7FFF)


def _per_element(block_values, n, block):
    return np.repeat(np.asarray(block_values), block)[:n]


# ------------------------------------------------------------------ scales (A2, A3)

def tensor_amax(x_bits) -> np.float32:
    """A = max |x| over the whole call tensor (exact). The NVFP4 global scale
    is per tensor ("the same global and block scales", §3.1, Fig. 4(a))."""
    x = _u16(x_bits)
    if x.size == 0:
        return _F32(0.0)
    return _abs_f32(x).max()


def nvfp4_global_scale(amax) -> np.float32:
    """S = fp32(2688 / A), 1 for A = 0, at most FLT_MAX (reading stated in the
    module docstring)."""
    a = _F32(amax)
    if a == 0:
        return _F32(1.0)
    with np.errstate(over="ignore"):
        s = NVFP4_GLOBAL_NUM / a
    return min(_F32(s), FLT_MAX)


def block_amax(x_bits, block) -> np.ndarray:
    """Per-block max |x| (float32)."""
    return _abs_f32(_u16(x_bits)).reshape(-1, block).max(axis=1)


def nvfp4_block_scales(x_bits, gscale) -> np.ndarray:
    """E4M3 scale byte per 16-element block: e = E4M3_RNE(min(fp32(fp32(a/6)*S), 448))."""
    a = block_amax(x_bits, 16)
    s = _F32(gscale)
    with np.errstate(over="ignore"):
        u = (a / _F32(6.0)).astype(_F32) * s
    u = np.minimum(u.astype(_F32), _F32(448.0))
    return e4m3_encode(u)


def nvfp4_block_factors(scale_bytes, gscale):
    """(d, r) per block from the E4M3 bytes and S: d = fp32(e/S),
    r = min(fp32(S/e), FLT_MAX); both 0 where e == 0."""
    e = e4m3_value(np.asarray(scale_bytes, dtype=np.uint8))
    s = _F32(gscale)
    zero = e == 0
    e_safe = np.where(zero, _F32(1.0), e).astype(_F32)
    with np.errstate(over="ignore", under="ignore"):
        d = (e_safe / s).astype(_F32)
        r = np.minimum((s / e_safe).astype(_F32), FLT_MAX)
    d = np.where(zero, _F32(0.0), d).astype(_F32)
    r = np.where(zero, _F32(0.0), r).astype(_F32)
    return d, r


def mxfp4_block_scales(x_bits) -> np.ndarray:
    """E8M0 byte per 32-element block: E + 127 with
    E = clamp(floor(log2 a) - 2, -127, 127), E = -127 for a == 0 (§4.3 names
    the format; the floor(log2) - 2 rule maps the block max into [4, 8))."""
    a = block_amax(x_bits, 32).astype(np.float64)
    e = np.full(a.shape, -127, dtype=np.int64)
    nz = a > 0
    e[nz] = np.clip(floor_log2(a[nz]) - 2, -127, 127)
    return (e + 127).astype(np.uint8)


def mxfp4_block_factors(scale_bytes):
    """(d, r) per block: d = 2^E, r = 2^-E, exact in float32 for E in [-127, 127]."""
    e = np.asarray(scale_bytes, dtype=np.int64) - 127
    d = np.ldexp(np.ones(e.shape, dtype=_F32), e.astype(np.int32)).astype(_F32)
    r = np.ldexp(np.ones(e.shape, dtype=_F32), (-e).astype(np.int32)).astype(_F32)
    return d, r


def block_factors(fmt, scale_bytes, gscale):
    if fmt == NVFP4:
        return nvfp4_block_factors(scale_bytes, gscale)
    if fmt == MXFP4:
        return mxfp4_block_factors(scale_bytes)
    raise ValueError("fmt")


def normalize(x_bits, r_block, block) -> np.ndarray:
    """t = fp32(|x| * r) for each element, r its block's encode factor. This
    is z = x / s of the paper's Algorithm 1 prose (§3.2 / Appendix), taken in
    magnitude; the sign is carried separately."""
    x = _u16(x_bits)
    r = _per_element(r_block, x.size, block).astype(_F32)
    with np.errstate(over="ignore", under="ignore"):
        return (_abs_f32(x) * r).astype(_F32)


# ------------------------------------------------------------------ E2M1 rounding (A1, A6)

def rtn(t) -> np.ndarray:
    """Round-to-nearest onto the E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}:
    the index of the nearest magnitude; equidistant -> the even index
    (mantissa 0); above 6 -> 6 (index 7). The paper's worked values: 2.51 -> 3
    and 2.49 -> 2 (§3.1, Fig. 4(a))."""
    t = np.asarray(t, dtype=_F32).astype(np.float64)
    dist = np.abs(t[:, None] - E2M1_F32.astype(np.float64)[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # Among equidistant magnitudes prefer an even index; there are at most two
    # candidates and they are adjacent, so exactly one of them is even.
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    k = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    k = np.where(t > 6.0, 7, k)
    return k.astype(np.uint8)


def bracket(t):
    """The adjacent E2M1 candidates {q-, q+} around t (BracketFP4, Algorithm 1
    prose; §3.1 "two neighboring normalized FP4 E2M1 codewords"):
    lo = max{k : v(k) < t}, hi = lo + 1; a single codeword lo = hi = k when t
    equals v(k); lo = hi = 7 when t >= 6."""
    t = np.asarray(t, dtype=_F32)
    v = E2M1_F32
    lo = np.zeros(t.shape, dtype=np.int64)
    for k in range(8):
        lo = np.where(v[k] < t, k, lo)
    hi = np.minimum(lo + 1, 7)
    exact = np.zeros(t.shape, dtype=bool)
    for k in range(8):
        exact |= t == v[k]
    for k in range(8):
        lo = np.where(t == v[k], k, lo)
    hi = np.where(exact, lo, hi)
    sat = t >= 6.0
    lo = np.where(sat, 7, lo)
    hi = np.where(sat, 7, hi)
    return lo.astype(np.uint8), hi.astype(np.uint8)


def reconstruct(t, c, b=1) -> np.ndarray:
    """Compact rollout reference (Reconstruct, Algorithm 1 prose): the E2M1
    magnitude nearest t whose low b bits of the 3-bit magnitude index equal c
    (b = 1: the mantissa bit; b = 3: the whole magnitude). Ties go to the
    larger magnitude. Returns the 3-bit index; the caller pairs it with the
    training sign."""
    t = np.asarray(t, dtype=_F32).astype(np.float64)
    c = np.asarray(c, dtype=np.int64)
    mask = (1 << b) - 1
    v = E2M1_F32.astype(np.float64)
    best_k = np.zeros(t.shape, dtype=np.int64)
    best_d = np.full(t.shape, np.inf)
    for k in range(8):                      # ascending, so "<=" keeps the larger on ties
        ok = (k & mask) == c
        dk = np.abs(v[k] - t)
        take = ok & (dk <= best_d)
        best_k = np.where(take, k, best_k)
        best_d = np.where(take, dk, best_d)
    return best_k.astype(np.uint8)


def signed_value(sign, k) -> np.ndarray:
    """(-1)^s * v(k) as float64."""
    v = E2M1_F32.astype(np.float64)[np.asarray(k, dtype=np.int64)]
    return np.where(np.asarray(sign) != 0, -v, v)


def select_full(lo, hi, s_t, s_r, k_r) -> np.ndarray:
    """Full-information TRACE selection (§3.1, "Key Design"; Eq. 2 lost in
    extraction, prose kept): of the two candidates, both carrying the training
    sign, take the one closer to the rollout codeword q_rollout. Ties cannot
    occur between two distinct adjacent candidates (q_rollout is a codeword)."""
    q_r = signed_value(s_r, k_r)
    d_lo = np.abs(signed_value(s_t, lo) - q_r)
    d_hi = np.abs(signed_value(s_t, hi) - q_r)
    return np.where(d_hi < d_lo, hi, lo).astype(np.uint8)


def select_compact(lo, hi, r_k) -> np.ndarray:
    """Compact selection: of the two candidates take the one whose magnitude is
    closer to the reconstructed reference v(r_k) (both carry the training
    sign, so magnitudes decide)."""
    v = E2M1_F32.astype(np.float64)
    ref = v[np.asarray(r_k, dtype=np.int64)]
    d_lo = np.abs(v[np.asarray(lo, dtype=np.int64)] - ref)
    d_hi = np.abs(v[np.asarray(hi, dtype=np.int64)] - ref)
    return np.where(d_hi < d_lo, hi, lo).astype(np.uint8)


def dequant(sign, k, d_block, block) -> np.ndarray:
    """y = (-1)^s * bf16(fp32(v(k) * d)) as bf16 bits (fake quantization
    output, §3.1 "Motivation": FP4 fake quantization in the forward pass)."""
    k = np.asarray(k, dtype=np.int64)
    d = _per_element(d_block, k.size, block).astype(_F32)
    with np.errstate(over="ignore", under="ignore"):
        mag = (E2M1_F32[k] * d).astype(_F32)
    bits = f32_to_bf16(mag)
    return (bits | (np.asarray(sign, dtype=np.uint16) << 15)).astype(np.uint16)


# ------------------------------------------------------------------ planes

def codes_of(sign, k) -> np.ndarray:
    """4-bit E2M1 code: sign << 3 | k."""
    return ((np.asarray(sign, dtype=np.uint8) << 3) | np.asarray(k, dtype=np.uint8)).astype(np.uint8)


def pack_codes(codes) -> np.ndarray:
    """Two codes per byte: element 2j in the low nibble, 2j + 1 in the high."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1, 2)
    return (c[:, 0] | (c[:, 1] << 4)).astype(np.uint8)


def unpack_codes(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    return np.stack([p & 0xF, p >> 4], axis=1).reshape(-1)


def pack_bits(bits) -> np.ndarray:
    """One bit per element, LSB first: element 8j + i is bit i of byte j."""
    b = np.asarray(bits, dtype=np.uint8).reshape(-1, 8)
    out = np.zeros(b.shape[0], dtype=np.uint8)
    for i in range(8):
        out |= (b[:, i] & 1) << i
    return out


def unpack_bits(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    return np.stack([(p >> i) & 1 for i in range(8)], axis=1).reshape(-1).astype(np.uint8)


def pack_low_bits(vals, b) -> np.ndarray:
    """b-bit fields, LSB first, as one bit string: element i occupies bits
    b*i .. b*i + b - 1 of the little-endian stream (b = 1: pack_bits; b = 2:
    four elements per byte; b = 3: eight elements per three bytes)."""
    v = np.asarray(vals, dtype=np.int64).reshape(-1)
    bitstream = np.zeros(v.size * b, dtype=np.uint8)
    for j in range(b):
        bitstream[j::b] = (v >> j) & 1
    return pack_bits(bitstream)


def unpack_low_bits(packed, b, n) -> np.ndarray:
    bitstream = unpack_bits(packed)[: n * b].astype(np.int64)
    out = np.zeros(n, dtype=np.int64)
    for j in range(b):
        out |= bitstream[j::b] << j
    return out.astype(np.uint8)


def guide_bytes(bits, n) -> int:
    """Bytes of a guidance plane for n elements: n * bits / 8 (bits 1..4)."""
    return n * bits // 8


# ------------------------------------------------------------------ the five calls

def _scales(fmt, x, gscale_in):
    """Scale bytes, S and A for one tensor (NVFP4: S from A unless supplied)."""
    if fmt == NVFP4:
        amax = tensor_amax(x)
        s = nvfp4_global_scale(amax) if gscale_in is None else _F32(gscale_in)
        return nvfp4_block_scales(x, s), s, amax
    if fmt == MXFP4:
        if gscale_in is not None:
            raise ValueError("MXFP4 has no global scale")
        return mxfp4_block_scales(x), None, None
    raise ValueError("fmt")


def quantize_rtn(fmt, x_bits, gscale=None):
    """Vanilla FP4 (fake) quantization of one tensor: own scales, RTN (§3.1).

    Returns dict(codes=packed u8[N/2], scales=u8[N/B], gscale=S or None,
    amax=A or None, y=bf16 bits[N], k=indices, sign=signs)."""
    x = _u16(x_bits)
    B = BLOCK[fmt]
    scales, s, amax = _scales(fmt, x, gscale)
    d, r = block_factors(fmt, scales, s)
    t = normalize(x, r, B)
    k = rtn(t)
    sg = _sign(x)
    return dict(codes=pack_codes(codes_of(sg, k)), scales=scales, gscale=s,
                amax=amax, y=dequant(sg, k, d, B), k=k, sign=sg)


def encode_guidance(fmt, bits, x_bits, gscale=None):
    """Rollout side: quantize with RTN and emit the guidance record (§3.2,
    "Key Design"; Algorithm 1 prose: packed low-bit rollout codes plus the
    rollout scales). bits=1 keeps the mantissa bit of each code (1 bit per
    element; with the amortized E4M3 scale 1.5 bits per element for NVFP4);
    bits=2 and 3 keep the low 2 or 3 bits of the magnitude index (Algorithm
    1's parameter b); bits=4 keeps the full signed code (the full-information
    record).

    Returns dict(guide, scales, gscale, amax, y) with guide = the packed low
    bits u8[N*bits/8] (bits 1..3, pack_low_bits) or the packed codes u8[N/2]
    (bits=4); y is the rollout's own fake-quantized output."""
    q = quantize_rtn(fmt, x_bits, gscale)
    if bits in (1, 2, 3):
        guide = pack_low_bits(q["k"] & ((1 << bits) - 1), bits)
    elif bits == 4:
        guide = q["codes"]
    else:
        raise ValueError("bits")
    return dict(guide=guide, scales=q["scales"], gscale=q["gscale"],
                amax=q["amax"], y=q["y"])


def train_normalized(fmt, x_bits, scales, gscale):
    """Training values under the rollout scales: (t, d per block, sign)."""
    x = _u16(x_bits)
    B = BLOCK[fmt]
    d, r = block_factors(fmt, scales, gscale)
    return normalize(x, r, B), d, _sign(x)


def decode_guidance(fmt, x_bits, guide, scales, gscale=None, bits=1):
    """Training side, compact record: Reconstruct the reference code of every
    element from the training value under the rollout scale and the rollout's
    low `bits` magnitude bits, with the training sign (Algorithm 1 prose).
    Returns packed reference codes u8[N/2]."""
    t, _, sg = train_normalized(fmt, x_bits, scales, gscale)
    c = unpack_low_bits(guide, bits, t.size)
    return pack_codes(codes_of(sg, reconstruct(t, c, bits)))


def guided_fake_quant(fmt, bits, x_bits, guide, scales, gscale=None):
    """Training side, rollout-guided rounding (§3.1 "Key Design"; Algorithm 1
    prose). Under the rollout scale, bracket t = |x| * r and pick:
    bits=0: RTN (the comparison q_RTN of the local guarantee);
    bits=1, 2, 3: the candidate nearest the reference reconstructed from the
    rollout's low `bits` magnitude bits;
    bits=4: the candidate nearest the exact rollout codeword.
    The output keeps the training sign and is dequantized with the rollout
    decode factor. Returns dict(y=bf16 bits[N], codes=packed u8[N/2], k)."""
    t, d, sg = train_normalized(fmt, x_bits, scales, gscale)
    B = BLOCK[fmt]
    if bits == 0:
        k = rtn(t)
    else:
        lo, hi = bracket(t)
        if bits in (1, 2, 3):
            c = unpack_low_bits(guide, bits, t.size)
            k = select_compact(lo, hi, reconstruct(t, c, bits))
        elif bits == 4:
            cr = unpack_codes(guide)[: t.size]
            k = select_full(lo, hi, sg, cr >> 3, cr & 7)
        else:
            raise ValueError("bits")
    return dict(y=dequant(sg, k, d, B), codes=pack_codes(codes_of(sg, k)), k=k)


def discrepancy_stats(x_t_bits, x_r_bits, y_t_bits, y_r_bits):
    """Sums behind the paper's discrepancy measures (§3.1, Eq. 1 lost in
    extraction; "Key Design", Fig. 4(b)): SB = sum (x_t - x_r)^2 over the bf16
    inputs, SF = sum (y_t - y_r)^2 over the FP4 outputs, and n. Then
    D_BF16 = SB / n, D_FP4 = SF / n and the relative excess
    (D_FP4 - D_BF16) / D_BF16 = (SF - SB) / SB. float64 here; the tests use
    exact rationals on small inputs."""
    xt = bf16_to_f32(_u16(x_t_bits)).astype(np.float64)
    xr = bf16_to_f32(_u16(x_r_bits)).astype(np.float64)
    yt = bf16_to_f32(_u16(y_t_bits)).astype(np.float64)
    yr = bf16_to_f32(_u16(y_r_bits)).astype(np.float64)
    sb = float(np.sum((xt - xr) ** 2))
    sf = float(np.sum((yt - yr) ** 2))
    return sb, sf, float(xt.size)


def code_position(codes) -> np.ndarray:
    """Position of an (unpacked) E2M1 code on the signed grid
    -6 < -4 < ... < -0.5 < 0 < 0.5 < ... < 6: the magnitude index with the
    code's sign (+0 and -0 are both 0), so adjacent codewords are one apart."""
    c = np.asarray(codes, dtype=np.int64)
    k = c & 7
    return np.where((c & 8) != 0, -k, k)


MISMATCH_BINS = 15          # distances 0..14 on the signed grid
MISMATCH_COUNTS = 2 * MISMATCH_BINS + 2


def mismatch_counts(codes_t, codes_r, codes_b):
    """Diagnostics of the mismatch between training and rollout codes
    (§3.2 "Key Design", Fig. 6: over 99% of mismatched values differ by one
    adjacent codebook entry; corrections toward lower codewords concentrate
    in deeper layers). Inputs are unpacked codes: the guided training codes,
    the rollout codes, and the training codes under RTN with the rollout
    scale (the vanilla baseline under the same candidate set). Returns
    int64[32]: [0..14] histogram of |p(t) - p(r)|; [15..29] histogram of
    |p(b) - p(r)|; [30] elements where the guided magnitude exceeds the RTN
    one; [31] elements where it is lower."""
    pt, pr, pb = code_position(codes_t), code_position(codes_r), code_position(codes_b)
    out = np.zeros(MISMATCH_COUNTS, dtype=np.int64)
    out[:MISMATCH_BINS] = np.bincount(np.abs(pt - pr), minlength=MISMATCH_BINS)[:MISMATCH_BINS]
    out[MISMATCH_BINS:2 * MISMATCH_BINS] = np.bincount(np.abs(pb - pr), minlength=MISMATCH_BINS)[:MISMATCH_BINS]
    kt = np.asarray(codes_t, dtype=np.int64) & 7
    kb = np.asarray(codes_b, dtype=np.int64) & 7
    out[2 * MISMATCH_BINS] = int(np.count_nonzero(kt > kb))
    out[2 * MISMATCH_BINS + 1] = int(np.count_nonzero(kt < kb))
    return out


def derived_metrics(sb, sf, n):
    """D_BF16, D_FP4, relative excess and D_act = ||Q_t(X_t) - Q_r(X_r)||_F.
    The relative excess is +inf for SB == 0 < SF and NaN for 0 / 0."""
    d_bf16 = sb / n if n else float("nan")
    d_fp4 = sf / n if n else float("nan")
    if sb > 0:
        rel = (sf - sb) / sb
    elif sf > 0:
        rel = float("inf")
    else:
        rel = float("nan")
    return dict(D_BF16=d_bf16, D_FP4=d_fp4, rel_excess=rel, D_act=float(np.sqrt(sf)))
