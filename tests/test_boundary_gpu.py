"""GPU parity where binary32 decides: normalized values t = fp32(|x| * r)
placed exactly on every E2M1 rounding boundary and around it.

The bf16 inputs of the other tests give t only on a coarse grid (8 mantissa
bits times the block factor), so boundaries are hit there only by chance. Here
every row is its own global-scale group with a supplied S (group_rows = 1,
gscale_in), chosen on the host with the oracle's formulas: a block maximum a
makes the E4M3 block scale exactly 1 (so r = fp32(S / 1) = S), and the members
are +-2^m, so t = 2^m * S is any binary32 value we like. The targets are each
E2M1 codeword, each RTN midpoint, the dead-zone edges of the 1-bit
Reconstruct (2.25, 4.5), the midpoints of the 2-bit Reconstruct (1, 1.75, 2.5,
3.75), each of these +-1..12 ulp, the saturation edge 6, values above it, and
binary32 subnormal t. Each member's rollout partner is one of the 16 signed
codewords, so guided rounding meets every (t, rollout code) pair of a row.

Every call of the path runs on these tensors (quantize_rtn, encode_guidance
with bits 1-4 on both sides, guided_fake_quant with bits 0-4 and the fused
statistics, decode_guidance with bits 1-3) and is compared with the oracle row
by row, bit for bit. Two layouts: 48 columns (one group per workgroup tile)
and 64 columns (several whole groups packed in a tile)."""

import numpy as np
import pytest
import torch

import precision_rl_nvfp4_amd as tq
from oracle import formats, fp4 as ofp4
from tests import _gpu as G

NV = tq.NVFP4
E4M3_ONE = 0x38
BASES = [0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75, 2.0, 2.25, 2.5, 3.0, 3.5, 3.75, 4.0, 4.5, 5.0, 6.0]
ULPS = 12
CODEWORDS = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float32)


def _targets():
    out = []
    for b in BASES:
        v = np.float32(b)
        lo = hi = v
        out.append(v)
        for _ in range(ULPS):
            lo = np.nextafter(lo, np.float32(0))
            hi = np.nextafter(hi, np.float32(np.inf))
            out += [lo, hi]
    out += [np.float32(v) for v in (6.5, 7.0, 8.0, 100.0, 1e-3)]
    out += [np.float32(2.0 ** -149), np.float32(2.0 ** -140), np.float32(2.0 ** -127), np.float32(2.0 ** -126)]
    return np.array(out, np.float32)


def _bf16(v):
    return formats.f32_to_bf16(np.array([v], np.float32))[0]


def _e_of(a_bits, S):
    blk = np.zeros(16, np.uint16)
    blk[0] = a_bits
    return int(ofp4.nvfp4_block_scales(blk, np.float32(S))[0])


def _row_params(t):
    """(S, member bits 2^m, block max bits a) with e(a, S) = 1 and, for t <= 6,
    a >= 2^m; None when no such a exists near 6 / S."""
    m = max(int(np.floor(np.log2(np.float64(t)))), -133) if t < 0.25 else 0
    S = np.float32(np.float64(t) / 2.0 ** m)
    x = _bf16(np.float32(2.0 ** m))
    assert formats.bf16_to_f32(np.array([x], np.uint16))[0] == np.float32(2.0 ** m)
    # the smallest bf16 a >= 6 / S with e = 1, so that no rollout member
    # (|x_r| <= 6 / S) exceeds it
    lim = 6.0 / np.float64(S)
    a0 = formats.f32_to_bf16(np.array([lim], np.float32))[0]
    for d in range(-2, 16):
        a = np.uint16(int(a0) + d)
        if formats.bf16_to_f32(np.array([a], np.uint16))[0] >= lim and _e_of(a, S) == E4M3_ONE:
            return S, x, a
    return None


def _build(cols):
    """Training and rollout tensors [rows, cols] plus the per-row S."""
    per_blk = 15
    nblk = cols // 16
    rows_t, rows_r, Ss, ts = [], [], [], []
    for t in _targets():
        p = _row_params(t)
        if p is None:
            continue
        S, x, a = p
        members = nblk * per_blk
        j = np.arange(members)
        sign_t = ((j // 16) & 1).astype(np.uint16) << 15
        code = j % 16
        k, sign_r = code & 7, (code >> 3).astype(np.uint16) << 15
        # rollout members: v(k) / S rounded toward zero, so |x_r| <= 6 / S <= a
        vr = (CODEWORDS[k].astype(np.float64) / np.float64(S)).astype(np.float32)
        vr_b = (vr.view(np.uint32) >> 16).astype(np.uint16)
        xt_m = (np.full(members, x, np.uint16) | sign_t).reshape(nblk, per_blk)
        xr_m = (vr_b | sign_r).reshape(nblk, per_blk)
        rt = np.zeros((nblk, 16), np.uint16)
        rr = np.zeros((nblk, 16), np.uint16)
        rt[:, 0] = a
        rr[:, 0] = a
        rt[:, 1:] = xt_m
        rr[:, 1:] = xr_m
        rows_t.append(rt.reshape(-1))
        rows_r.append(rr.reshape(-1))
        Ss.append(S)
        ts.append(t)
    return np.stack(rows_t), np.stack(rows_r), np.array(Ss, np.float32), np.array(ts, np.float32)


def _gdev(S):
    return torch.from_numpy(np.stack([S, np.zeros_like(S)], 1).copy()).to(G.DEV)


def test_sweep_construction_hits_the_targets():
    """Host-side check of the construction itself (the oracle's block scale
    and normalization): the rollout blocks all get e = 1 and the training
    members' t under the rollout scale is exactly the target."""
    xt, xr, S, ts = _build(48)
    assert len(ts) == len(_targets())
    for i in range(len(ts)):
        sc = ofp4.nvfp4_block_scales(xr[i], S[i])
        assert np.all(sc == E4M3_ONE), (i, ts[i], sc)
        _, r = ofp4.nvfp4_block_factors(sc, S[i])
        t = ofp4.normalize(xt[i], r, 16)
        members = np.ones(48, bool)
        members[0::16] = False
        assert np.all(t[members] == ts[i]), (i, ts[i])


@pytest.mark.gpu
@pytest.mark.parametrize("cols", [48, 64])
def test_boundary_sweep(cols):
    xt, xr, S, ts = _build(cols)
    rows = xt.shape[0]
    G.say(f"boundary sweep: {rows} rows x {cols} columns, one supplied S per row")
    dt, dr = G.to_dev(xt.reshape(-1), rows, cols), G.to_dev(xr.reshape(-1), rows, cols)
    gs = _gdev(S)
    q = tq.quantize_rtn(dt, NV, gscale=gs, group_rows=1)
    enc_t = {b: tq.encode_guidance(dt, NV, b, gscale=gs, with_y=True, group_rows=1) for b in (1, 2, 3, 4)}
    rec = {b: tq.encode_guidance(dr, NV, b, gscale=gs, with_y=True, group_rows=1) for b in (1, 2, 3, 4)}
    guided = {b: tq.guided_fake_quant(dt, rec[max(b, 1) if b else 4], bits=b, with_codes=True) for b in range(5)}
    stats = {b: tq.guided_fake_quant_stats(dt, dr, rec[b], with_codes=True) for b in (1, 4)}
    dec = {b: tq.decode_guidance(dt, rec[b]) for b in (1, 2, 3)}
    torch.cuda.synchronize()
    B = 16

    def rowv(t, i):
        return G.u8(t).reshape(rows, -1)[i] if t.dtype == torch.uint8 else G.bits_of(t).reshape(rows, -1)[i]

    for i in range(rows):
        bt, br, s = xt[i], xr[i], S[i]
        oq = ofp4.quantize_rtn(NV, bt, s)
        G.assert_same(rowv(q.codes, i), oq["codes"], f"rtn codes t={ts[i]!r}")
        G.assert_same(rowv(q.scales, i), oq["scales"], f"rtn scales t={ts[i]!r}")
        G.assert_same(rowv(q.y, i), oq["y"], f"rtn y t={ts[i]!r}")
        orec = {}
        for b in (1, 2, 3, 4):
            o = ofp4.encode_guidance(NV, b, bt, s)
            G.assert_same(rowv(enc_t[b].guide, i), o["guide"], f"encode bits={b} t={ts[i]!r}")
            G.assert_same(rowv(enc_t[b].y, i), o["y"], f"encode y bits={b} t={ts[i]!r}")
            orec[b] = ofp4.encode_guidance(NV, b, br, s)
            G.assert_same(rowv(rec[b].guide, i), orec[b]["guide"], f"rollout record bits={b} t={ts[i]!r}")
            G.assert_same(rowv(rec[b].scales, i), orec[b]["scales"], f"rollout scales t={ts[i]!r}")
        for b in range(5):
            r = orec[b if b else 4]
            og = ofp4.guided_fake_quant(NV, b, bt, r["guide"] if b else None, r["scales"], s)
            y, codes = guided[b]
            G.assert_same(rowv(y, i), og["y"], f"guided y bits={b} t={ts[i]!r}")
            G.assert_same(rowv(codes, i), og["codes"], f"guided codes bits={b} t={ts[i]!r}")
            if b in stats:
                G.assert_same(rowv(stats[b][0], i), og["y"], f"guided y (stats) bits={b} t={ts[i]!r}")
                G.assert_same(rowv(stats[b][1], i), og["codes"], f"guided codes (stats) bits={b} t={ts[i]!r}")
        for b in (1, 2, 3):
            od = ofp4.decode_guidance(NV, bt, orec[b]["guide"], orec[b]["scales"], s, bits=b)
            G.assert_same(rowv(dec[b], i), od, f"decode bits={b} t={ts[i]!r}")
