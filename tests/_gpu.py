"""Helpers shared by the GPU parity tests: move bit patterns between numpy
(oracle side) and torch device tensors (library side), and compare the
library's outputs with the oracle's element by element."""

from __future__ import annotations

import sys

import numpy as np
import torch

import precision_rl_nvfp4_amd as tq
from oracle import fp4 as ofp4

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray, rows: int, cols: int) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).reshape(rows, cols).to(DEV)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy().reshape(-1)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.float32).reshape(-1)


def first_diff(a, b):
    a = np.asarray(a).reshape(-1)
    b = np.asarray(b).reshape(-1)
    if a.shape != b.shape:
        return f"shape {a.shape} vs {b.shape}"
    idx = np.flatnonzero(a != b)
    if idx.size == 0:
        return None
    i = idx[0]
    return f"{idx.size} mismatches; first at {i}: got {a[i]!r}, want {b[i]!r}"


def assert_same(got, want, what):
    d = first_diff(got, want)
    assert d is None, f"{what}: {d}"


def fmt_of(name):
    return tq.NVFP4 if name == "nvfp4" else tq.MXFP4


def check_quantize(xb: np.ndarray, rows: int, cols: int, fmt: int, gscale=None, with_y=True):
    """quantize_rtn on the GPU vs the oracle; returns the oracle result."""
    x = to_dev(xb, rows, cols)
    g_in = None if gscale is None else torch.tensor([gscale, 0.0], dtype=torch.float32, device=DEV)
    q = tq.quantize_rtn(x, fmt, gscale=g_in, with_y=with_y)
    o = ofp4.quantize_rtn(fmt, xb, gscale)
    assert_same(u8(q.codes), o["codes"], "codes")
    assert_same(u8(q.scales), o["scales"], "scales")
    if with_y:
        assert_same(bits_of(q.y), o["y"], "y")
    if fmt == tq.NVFP4 and gscale is None:
        g = f32(q.gscale)
        assert g[0] == o["gscale"], (g, o["gscale"])
        assert g[1] == o["amax"], (g, o["amax"])
    return o


def check_encode(xb, rows, cols, fmt, bits, with_y=True):
    x = to_dev(xb, rows, cols)
    g = tq.encode_guidance(x, fmt, bits, with_y=with_y)
    o = ofp4.encode_guidance(fmt, bits, xb)
    assert_same(u8(g.guide), o["guide"], f"guide bits={bits}")
    assert_same(u8(g.scales), o["scales"], "scales")
    if with_y:
        assert_same(bits_of(g.y), o["y"], "rollout y")
    if fmt == tq.NVFP4:
        assert f32(g.gscale)[0] == o["gscale"]
    return g, o


def check_guided(xt_bits, xr_bits, rows, cols, fmt, bits, with_codes=True):
    """Encode the rollout (bits 1 or 4; bits 0 uses a bits=4 record's scales),
    then guided rounding of the training tensor, GPU vs oracle."""
    rec_bits = 4 if bits == 0 else bits
    xr = to_dev(xr_bits, rows, cols)
    xt = to_dev(xt_bits, rows, cols)
    g = tq.encode_guidance(xr, fmt, rec_bits, with_y=True)
    y, codes = tq.guided_fake_quant(xt, g, bits=bits, with_codes=with_codes)
    o_enc = ofp4.encode_guidance(fmt, rec_bits, xr_bits)
    o = ofp4.guided_fake_quant(fmt, bits, xt_bits, o_enc["guide"], o_enc["scales"], o_enc["gscale"])
    assert_same(u8(g.guide), o_enc["guide"], "guide")
    assert_same(bits_of(y), o["y"], f"guided y bits={bits}")
    if with_codes:
        assert_same(u8(codes), o["codes"], f"guided codes bits={bits}")
    return g, y, o_enc, o


def check_decode(xt_bits, xr_bits, rows, cols, fmt):
    xr = to_dev(xr_bits, rows, cols)
    xt = to_dev(xt_bits, rows, cols)
    g = tq.encode_guidance(xr, fmt, 1)
    ref = tq.decode_guidance(xt, g)
    o_enc = ofp4.encode_guidance(fmt, 1, xr_bits)
    o = ofp4.decode_guidance(fmt, xt_bits, o_enc["guide"], o_enc["scales"], o_enc["gscale"])
    assert_same(u8(ref), o, "reference codes")
