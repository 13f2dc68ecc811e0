"""Helpers shared by the GPU parity tests: move bit patterns between numpy
(oracle side) and torch device tensors (library side), run the oracle group
by group (a grouped call quantizes each group of rows as its own tensor), and
compare the library's outputs with the oracle's element by element."""

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


def rel_close(got, want, tol=1e-6):
    return abs(got - want) <= tol * abs(want) or got == want


# ---------------------------------------------------------------- grouped oracle

def n_groups(rows, group_rows):
    return rows // group_rows if group_rows else 1


def group_slices(n, G, fmt, plane_bits):
    """Element, plane-byte and scale-byte slices of each of G equal groups
    (plane_bits: bits per element of the plane, 1..4)."""
    ng = n // G
    B = ofp4.BLOCK[fmt]
    pb = lambda e: e * plane_bits // 8  # noqa: E731
    return [(slice(g * ng, (g + 1) * ng), slice(pb(g * ng), pb((g + 1) * ng)),
             slice(g * ng // B, (g + 1) * ng // B)) for g in range(G)]


def oracle_quantize(fmt, xb, rows, group_rows=0, gscale=None):
    """quantize_rtn of the oracle, applied per group. gscale: one S for every
    group or an array of per-group S."""
    G = n_groups(rows, group_rows)
    parts = []
    for g, (es, _, _) in enumerate(group_slices(xb.size, G, fmt, 4)):
        s = None if gscale is None else np.asarray(gscale, np.float32).reshape(-1)[g % np.size(gscale)]
        parts.append(ofp4.quantize_rtn(fmt, xb[es], s))
    cat = lambda k: np.concatenate([p[k] for p in parts]) if parts else np.zeros(0)
    out = {k: cat(k) for k in ("codes", "scales", "y", "k", "sign")}
    out["gscale"] = np.array([p["gscale"] for p in parts], np.float32) if fmt == ofp4.NVFP4 else None
    out["amax"] = np.array([p["amax"] for p in parts], np.float32) if fmt == ofp4.NVFP4 else None
    return out


def oracle_encode(fmt, bits, xb, rows, group_rows=0):
    G = n_groups(rows, group_rows)
    parts = [ofp4.encode_guidance(fmt, bits, xb[es])
             for es, _, _ in group_slices(xb.size, G, fmt, bits)]
    out = {k: np.concatenate([p[k] for p in parts]) for k in ("guide", "scales", "y")}
    out["gscale"] = np.array([p["gscale"] for p in parts], np.float32) if fmt == ofp4.NVFP4 else None
    return out


def oracle_guided(fmt, bits, xt, enc, rows, group_rows=0):
    """guided_fake_quant of the oracle per group against an oracle record."""
    G = n_groups(rows, group_rows)
    ys, cs = [], []
    for g, (es, ps, ss) in enumerate(group_slices(xt.size, G, fmt, max(bits, 1))):
        guide = None if bits == 0 else enc["guide"][ps]
        S = None if enc["gscale"] is None else enc["gscale"][g]
        o = ofp4.guided_fake_quant(fmt, bits, xt[es], guide, enc["scales"][ss], S)
        ys.append(o["y"])
        cs.append(o["codes"])
    return {"y": np.concatenate(ys), "codes": np.concatenate(cs)}


def oracle_decode(fmt, xt, enc, rows, group_rows=0, bits=1):
    G = n_groups(rows, group_rows)
    out = []
    for g, (es, ps, ss) in enumerate(group_slices(xt.size, G, fmt, bits)):
        S = None if enc["gscale"] is None else enc["gscale"][g]
        out.append(ofp4.decode_guidance(fmt, xt[es], enc["guide"][ps], enc["scales"][ss], S, bits))
    return np.concatenate(out)


# ---------------------------------------------------------------- checks

def check_quantize(xb: np.ndarray, rows: int, cols: int, fmt: int, gscale=None, with_y=True,
                   group_rows=0):
    """quantize_rtn on the GPU vs the oracle; returns the oracle result."""
    x = to_dev(xb, rows, cols)
    G = n_groups(rows, group_rows)
    g_in = None
    if gscale is not None:
        s = np.broadcast_to(np.asarray(gscale, np.float32).reshape(-1), (G,))
        g_in = torch.from_numpy(np.stack([s, np.zeros(G, np.float32)], 1).copy()).to(DEV)
    q = tq.quantize_rtn(x, fmt, gscale=g_in, with_y=with_y, group_rows=group_rows)
    o = oracle_quantize(fmt, xb, rows, group_rows, gscale)
    assert_same(u8(q.codes), o["codes"], "codes")
    assert_same(u8(q.scales), o["scales"], "scales")
    if with_y:
        assert_same(bits_of(q.y), o["y"], "y")
    if fmt == tq.NVFP4 and gscale is None:
        g = f32(q.gscale).reshape(G, 2)
        assert_same(g[:, 0], o["gscale"], "S")
        assert_same(g[:, 1], o["amax"], "A")
    return o


def check_encode(xb, rows, cols, fmt, bits, with_y=True, group_rows=0):
    x = to_dev(xb, rows, cols)
    g = tq.encode_guidance(x, fmt, bits, with_y=with_y, group_rows=group_rows)
    o = oracle_encode(fmt, bits, xb, rows, group_rows)
    assert_same(u8(g.guide), o["guide"], f"guide bits={bits}")
    assert_same(u8(g.scales), o["scales"], "scales")
    if with_y:
        assert_same(bits_of(g.y), o["y"], "rollout y")
    if fmt == tq.NVFP4:
        assert_same(f32(g.gscale).reshape(-1, 2)[:, 0], o["gscale"], "S")
    return g, o


def check_guided(xt_bits, xr_bits, rows, cols, fmt, bits, with_codes=True, group_rows=0):
    """Encode the rollout (bits 1 or 4; bits 0 uses a bits=4 record's scales),
    then guided rounding of the training tensor, GPU vs oracle."""
    rec_bits = 4 if bits == 0 else bits
    xr = to_dev(xr_bits, rows, cols)
    xt = to_dev(xt_bits, rows, cols)
    g = tq.encode_guidance(xr, fmt, rec_bits, with_y=True, group_rows=group_rows)
    y, codes = tq.guided_fake_quant(xt, g, bits=bits, with_codes=with_codes)
    o_enc = oracle_encode(fmt, rec_bits, xr_bits, rows, group_rows)
    o = oracle_guided(fmt, bits, xt_bits, o_enc, rows, group_rows)
    assert_same(u8(g.guide), o_enc["guide"], "guide")
    assert_same(bits_of(y), o["y"], f"guided y bits={bits}")
    if with_codes:
        assert_same(u8(codes), o["codes"], f"guided codes bits={bits}")
    return g, y, o_enc, o


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """uint8[N/2] code plane -> uint8[N] codes (element 2i in the low nibble)."""
    p = np.asarray(packed, np.uint8).reshape(-1)
    out = np.empty(2 * p.size, np.uint8)
    out[0::2] = p & 15
    out[1::2] = p >> 4
    return out


def oracle_mismatch(fmt, bits, xt_bits, xr_bits, rows, group_rows, o_guided):
    """The oracle's mismatch counts for a guided result: rollout codes from a
    full-code (bits=4) record of the rollout, RTN codes of the training input
    under the same rollout scales (guided with bits=0)."""
    enc4 = oracle_encode(fmt, 4, xr_bits, rows, group_rows)
    rtn = o_guided if bits == 0 else oracle_guided(fmt, 0, xt_bits, enc4, rows, group_rows)
    return ofp4.mismatch_counts(unpack_codes(o_guided["codes"]), unpack_codes(enc4["guide"]),
                                unpack_codes(rtn["codes"]))


CHUNK_ELEMS = 1 << 21   # host-side chunk of the full-size checks (keeps numpy's buffers reused)


def oracle_plane_counts(codes_t: torch.Tensor, codes_r: torch.Tensor, codes_b: torch.Tensor,
                        step: int = CHUNK_ELEMS) -> np.ndarray:
    """The oracle's mismatch counts (oracle.fp4.mismatch_counts) over three
    packed device code planes of any size, chunk by chunk on the CPU: the
    guided codes, the rollout codes and the RTN codes under the rollout scales."""
    out = np.zeros(ofp4.MISMATCH_COUNTS, np.int64)
    a, b, c = codes_t.reshape(-1), codes_r.reshape(-1), codes_b.reshape(-1)
    half = step // 2
    for s0 in range(0, a.numel(), half):
        out += ofp4.mismatch_counts(ofp4.unpack_codes(u8(a[s0:s0 + half])), ofp4.unpack_codes(u8(b[s0:s0 + half])),
                                    ofp4.unpack_codes(u8(c[s0:s0 + half])))
    return out


def oracle_plane_sums(x_t: torch.Tensor, x_r: torch.Tensor, y_t: torch.Tensor, y_r: torch.Tensor,
                      step: int = CHUNK_ELEMS):
    """The oracle's discrepancy sums (oracle.fp4.discrepancy_stats, float64)
    over four device bf16 tensors of any size, chunk by chunk on the CPU:
    (SB, SF, n)."""
    fl = [t.reshape(-1) for t in (x_t, x_r, y_t, y_r)]
    sb = sf = n = 0.0
    for s0 in range(0, fl[0].numel(), step):
        a, b, c = ofp4.discrepancy_stats(*(bits_of(t[s0:s0 + step]) for t in fl))
        sb, sf, n = sb + a, sf + b, n + c
    return sb, sf, n


def check_guided_stats(xt_bits, xr_bits, rows, cols, fmt, bits, group_rows=0, tol=1e-6):
    """guided_fake_quant_stats: y and codes bit-exact; {SB, SF, n} within tol
    of the oracle's sums over (x_t, x_r, guided y, rollout y); the mismatch
    counts exactly the oracle's; a call without counts gives the same y, codes
    and sums bit for bit."""
    rec_bits = 4 if bits == 0 else bits
    xr = to_dev(xr_bits, rows, cols)
    xt = to_dev(xt_bits, rows, cols)
    g = tq.encode_guidance(xr, fmt, rec_bits, with_y=False, group_rows=group_rows)
    y, codes, acc, counts = tq.guided_fake_quant_stats(xt, xr, g, bits=bits, with_codes=True,
                                                       mismatch=True)
    y2, codes2, acc2 = tq.guided_fake_quant_stats(xt, xr, g, bits=bits, with_codes=True)
    o_enc = oracle_encode(fmt, rec_bits, xr_bits, rows, group_rows)
    o = oracle_guided(fmt, bits, xt_bits, o_enc, rows, group_rows)
    assert_same(bits_of(y), o["y"], f"guided y (stats) bits={bits}")
    assert_same(u8(codes), o["codes"], f"guided codes (stats) bits={bits}")
    assert_same(bits_of(y2), o["y"], f"guided y (stats, no counts) bits={bits}")
    assert_same(u8(codes2), o["codes"], f"guided codes (stats, no counts) bits={bits}")
    sb, sf, n = ofp4.discrepancy_stats(xt_bits, xr_bits, o["y"], o_enc["y"])
    a = acc.cpu().numpy()
    assert np.array_equal(a, acc2.cpu().numpy()), (a, acc2)
    assert a[2] == n, (a, n)
    assert rel_close(a[0], sb, tol), ("SB", a[0], sb)
    assert rel_close(a[1], sf, tol), ("SF", a[1], sf)
    want = oracle_mismatch(fmt, bits, xt_bits, xr_bits, rows, group_rows, o)
    assert_same(counts.cpu().numpy(), want, f"mismatch counts bits={bits}")
    return a, (sb, sf, n)


def check_decode(xt_bits, xr_bits, rows, cols, fmt, group_rows=0, bits=1):
    xr = to_dev(xr_bits, rows, cols)
    xt = to_dev(xt_bits, rows, cols)
    g = tq.encode_guidance(xr, fmt, bits, group_rows=group_rows)
    ref = tq.decode_guidance(xt, g)
    o_enc = oracle_encode(fmt, bits, xr_bits, rows, group_rows)
    o = oracle_decode(fmt, xt_bits, o_enc, rows, group_rows, bits)
    assert_same(u8(g.guide), o_enc["guide"], f"guide bits={bits}")
    assert_same(u8(ref), o, f"reference codes bits={bits}")
