"""GPU parity: every entry point against the CPU oracle, bit for bit, on
seeded inputs at sizes the oracle finishes in seconds. Sizes span several
workgroup tiles (8,192 elements each) and end in a ragged tail.

The statistics are compared within 1e-6 relative (the oracle sums in float64
in a different order)."""

import numpy as np
import pytest
import torch

import precision_rl_nvfp4_amd as tq
from precision_rl_nvfp4_amd import _abi
import synthetic as syn
from oracle import formats, fp4 as ofp4
from tests import _gpu as G

pytestmark = pytest.mark.gpu

NV, MX = tq.NVFP4, tq.MXFP4


def _pair(rows, cols, seed, mx=False):
    if mx:
        xt, xr = syn.mxfp4_pair(rows=rows, cols=cols, frac=0.01)
    else:
        xt, xr = syn.activation_pair(rows, cols, (90, seed))
    return syn.bits_u16(xt), syn.bits_u16(xr)


SHAPES = [  # (rows, cols): one block, sub-tile, ragged multi-tile, tiny workload, KV rows
    (1, 32), (7, 96), (37, 2048), (256, 2048), (333, 256),
]


@pytest.mark.parametrize("fmt", [NV, MX])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_quantize_rtn(fmt, rows, cols):
    G.say(f"quantize_rtn fmt={fmt} shape=({rows},{cols})")
    xt, _ = _pair(rows, cols, rows, mx=(fmt == MX and cols % 32 == 0))
    G.check_quantize(xt, rows, cols, fmt)


@pytest.mark.parametrize("fmt", [NV, MX])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_encode_guidance(fmt, bits, rows, cols):
    G.say(f"encode_guidance fmt={fmt} bits={bits} shape=({rows},{cols})")
    _, xr = _pair(rows, cols, rows + 1, mx=(fmt == MX))
    G.check_encode(xr, rows, cols, fmt, bits)


@pytest.mark.parametrize("fmt", [NV, MX])
@pytest.mark.parametrize("bits", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_guided_fake_quant(fmt, bits, rows, cols):
    G.say(f"guided_fake_quant fmt={fmt} bits={bits} shape=({rows},{cols})")
    xt, xr = _pair(rows, cols, rows + 2, mx=(fmt == MX))
    G.check_guided(xt, xr, rows, cols, fmt, bits, with_codes=True)
    G.check_guided(xt, xr, rows, cols, fmt, bits, with_codes=False)


@pytest.mark.parametrize("fmt", [NV, MX])
@pytest.mark.parametrize("bits", [1, 2, 3])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_decode_guidance(fmt, bits, rows, cols):
    G.say(f"decode_guidance fmt={fmt} bits={bits} shape=({rows},{cols})")
    xt, xr = _pair(rows, cols, rows + 3, mx=(fmt == MX))
    G.check_decode(xt, xr, rows, cols, fmt, bits=bits)


def test_quantize_without_y_and_with_given_scale():
    G.say("quantize_rtn given S / no y")
    xt, _ = _pair(64, 2048, 5)
    G.check_quantize(xt, 64, 2048, NV, with_y=False)
    for s in (1.0, 0.37, 1e-3, 3.0e4):
        G.check_quantize(xt, 64, 2048, NV, gscale=np.float32(s))


def test_empty_tensors():
    G.say("empty tensors")
    x = torch.empty(0, 2048, dtype=torch.bfloat16, device=G.DEV)
    q = tq.quantize_rtn(x, NV)
    assert G.f32(q.gscale).tolist() == [1.0, 0.0]
    g = tq.encode_guidance(x, MX, 1)
    y, c = tq.guided_fake_quant(x, g, with_codes=True)
    assert y.numel() == 0 and c.numel() == 0
    acc = tq.discrepancy_stats(x, x, x, x)
    assert acc.cpu().tolist() == [0.0, 0.0, 0.0]
    gn = tq.encode_guidance(x, NV, 1)
    y, _, acc = tq.guided_fake_quant_stats(x, x, gn)
    assert y.numel() == 0 and acc.cpu().tolist() == [0.0, 0.0, 0.0]
    # zero-width rows in groups: every group gets S = 1, A = 0
    z = torch.empty(6, 0, dtype=torch.bfloat16, device=G.DEV)
    q = tq.quantize_rtn(z, NV, group_rows=2)
    assert G.f32(q.gscale).tolist() == [1.0, 0.0] * 3


def _edge_tensor():
    """Blocks that exercise the scale corner cases: zero blocks, E4M3
    subnormal and zero scales next to a huge anchor, signed zeros, exact
    codewords, the largest bf16 values."""
    f = np.zeros((16, 64), np.float32)
    f[0, 0] = 3.0e38                         # tensor amax near the bf16 top
    f[1, :16] = np.linspace(-1e34, 1e34, 16)  # scale e in the subnormal range
    f[1, 16:32] = 1e33                        # e = 0: zero block
    f[2, :] = -0.0
    f[3, :16] = np.array([6, 4, 3, 2, 1.5, 1, .5, 0, -6, -4, -3, -2, -1.5, -1, -.5, -0.0]) * 1e36
    f[4, :] = np.linspace(-3e38, 3e38, 64)
    f[5, :32] = 2.0 ** -133                  # bf16 subnormals
    b = formats.f32_to_bf16(f)
    b[2, :] = 0x8000
    b[5, 32:] = np.arange(1, 33, dtype=np.uint16)   # more subnormal patterns
    return b.reshape(-1)


@pytest.mark.parametrize("fmt", [NV, MX])
def test_scale_corner_cases(fmt):
    G.say(f"scale corner cases fmt={fmt}")
    b = _edge_tensor()
    G.check_quantize(b, 16, 64, fmt)
    for bits in (1, 4):
        G.check_encode(b, 16, 64, fmt, bits)
    b2 = b.copy()
    b2[::3] ^= 0x0001                        # perturb the training side a little
    for bits in (0, 1, 4):
        G.check_guided(b2, b, 16, 64, fmt, bits)
    G.check_decode(b2, b, 16, 64, fmt)


def test_tiny_amax_clamps_global_scale():
    G.say("tiny amax")
    b = np.zeros(64, np.uint16)
    b[:8] = np.arange(1, 9)                   # largest value is the 8th bf16 subnormal
    G.check_quantize(b, 2, 32, NV)
    o = ofp4.quantize_rtn(NV, b)
    assert o["gscale"] == formats.FLT_MAX


def _enumeration_members():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = formats.bf16_to_f32(bits)
    return bits[np.isfinite(f) & (np.abs(f) <= 6.0)]


ROLLOUT_CODEWORDS = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6], np.float32)


def _members_tensor(members_t, members_r):
    """Rows of 32 elements: row 0 is the tensor anchor [2688, 0, ...] (NVFP4:
    A = 2688, S = 1); every other row holds two 16-element blocks, each with
    6 at its first position (NVFP4 e = 1, so d = r = 1; MXFP4 E = 0 for the
    32-element block) and 15 members. Returns (xt, xr, rows)."""
    per = 15
    nblk = -(-members_t.size // per)
    nblk += nblk % 2                          # whole rows of two blocks
    six = formats.f32_to_bf16(np.array([6.0], np.float32))[0]
    out = []
    for members in (members_t, members_r):
        x = np.zeros((nblk, 16), np.uint16)
        x[:, 0] = six
        flat = np.zeros(nblk * per, np.uint16)
        flat[: members.size] = members
        x[:, 1:] = flat.reshape(nblk, per)
        head = np.zeros(32, np.uint16)
        head[0] = formats.f32_to_bf16(np.array([2688.0], np.float32))[0]
        out.append(np.concatenate([head, x.reshape(-1)]))
    rows = out[0].size // 32
    return out[0], out[1], rows


def test_enumerate_bf16_members_unit_scale():
    """Every finite bf16 value with |x| <= 6 as a non-max block member under
    S = 1, e = 1 (and under MXFP4, E = 0): quantize_rtn and encode_guidance,
    GPU vs oracle."""
    G.say("enumeration: block members, own scales")
    members = _enumeration_members()
    xb, _, rows = _members_tensor(members, members)
    for fmt in (NV, MX):
        G.check_quantize(xb, rows, 32, fmt)
        for bits in (1, 2, 3, 4):
            G.check_encode(xb, rows, 32, fmt, bits)


@pytest.mark.parametrize("fmt", [NV, MX])
def test_enumerate_bf16_train_values_all_rollout_codes(fmt):
    """The whole training-side pipeline, exhaustively: every finite bf16 value
    (65,280 of them, so t = |x| covers every bf16 magnitude, the saturated
    range above 6 included) paired with each of the 16 signed rollout
    codewords, under unit rollout scales. Guided rounding with records of
    every width (bits 0 to 4) and Reconstruct (bits 1 to 3), GPU vs oracle,
    bit for bit."""
    G.say(f"enumeration: every bf16 training value x 16 rollout codes, fmt={fmt}")
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = allb[np.isfinite(formats.bf16_to_f32(allb))]
    assert finite.size == 65280
    train = np.repeat(finite, 16)
    roll = np.tile(formats.f32_to_bf16(ROLLOUT_CODEWORDS), finite.size)
    xt, xr, rows = _members_tensor(train, roll)
    for bits in (0, 1, 2, 3, 4):
        G.check_guided(xt, xr, rows, 32, fmt, bits)
    for bits in (1, 2, 3):
        G.check_decode(xt, xr, rows, 32, fmt, bits=bits)


def test_enumerate_bf16_block_max():
    """Every positive finite bf16 value as the max of its block, under three
    tensor anchors (the amax sets S): E4M3 normal, subnormal and zero scales,
    and the FLT_MAX clamp of S all occur."""
    G.say("enumeration: block max")
    pos = np.arange(1, 0x7F80, dtype=np.uint16)
    blocks = np.zeros((pos.size, 16), np.uint16)
    blocks[:, 0] = pos
    blocks[:, 1] = pos >> 1                     # a smaller member
    blocks[:, 2] = (pos - 1) | 0x8000           # a negative member
    for anchor in (0x7F7F, 0x4F00, 0x3F80):     # ~3.4e38, 2^31, 1.0
        keep = pos <= anchor
        xb = np.concatenate([[anchor], np.zeros(15, np.uint16), blocks[keep].reshape(-1)]).astype(np.uint16)
        pad = (-xb.size) % 32
        xb = np.concatenate([xb, np.zeros(pad, np.uint16)])
        rows = xb.size // 32
        G.check_quantize(xb, rows, 32, NV)
        G.check_quantize(xb, rows, 32, MX)


def test_guided_guarantee_on_gpu_outputs():
    """§3.1: on every element, |y_guided - y_r| <= |y_RTN(rollout scale) - y_r|
    with full-information guidance."""
    G.say("guarantee on GPU outputs")
    xt, xr = _pair(256, 2048, 77)
    t, r = G.to_dev(xt, 256, 2048), G.to_dev(xr, 256, 2048)
    g = tq.encode_guidance(r, NV, 4, with_y=True)
    yg, _ = tq.guided_fake_quant(t, g, bits=4)
    yn, _ = tq.guided_fake_quant(t, g, bits=0)
    dg = (yg.float() - g.y.float()).abs()
    dn = (yn.float() - g.y.float()).abs()
    assert bool((dg <= dn).all())
    assert float(dg.sum()) < float(dn.sum())


def test_stats_vs_oracle_and_deterministic():
    G.say("discrepancy_stats")
    for rows, cols in [(1, 16), (37, 2048), (256, 2048), (4096, 2048)]:
        xt, xr = _pair(rows, cols, 11)
        t, r = G.to_dev(xt, rows, cols), G.to_dev(xr, rows, cols)
        q_t = tq.quantize_rtn(t, NV)
        q_r = tq.quantize_rtn(r, NV)
        acc = tq.discrepancy_stats(t, r, q_t.y, q_r.y)
        acc2 = tq.discrepancy_stats(t, r, q_t.y, q_r.y)
        assert torch.equal(acc, acc2)
        sb, sf, n = ofp4.discrepancy_stats(xt, xr, G.bits_of(q_t.y), G.bits_of(q_r.y))
        a = acc.cpu().numpy()
        assert a[2] == n
        assert abs(a[0] - sb) <= 1e-6 * abs(sb)
        assert abs(a[1] - sf) <= 1e-6 * abs(sf)
        # accumulate over two halves equals one call
        half = rows * cols // 2
        if half % 8 == 0 and half > 0:
            fl = [v.reshape(-1) for v in (t, r, q_t.y, q_r.y)]
            acc3 = tq.discrepancy_stats(*(v[:half] for v in fl))
            tq.discrepancy_stats(*(v[half:] for v in fl), acc=acc3, accumulate=True)
            b = acc3.cpu().numpy()
            assert b[2] == n and abs(b[0] - sb) <= 1e-6 * sb and abs(b[1] - sf) <= 1e-6 * sf


def test_stats_ragged_lengths():
    G.say("discrepancy_stats ragged")
    rng = np.random.default_rng(3)
    for n in (1, 7, 9, 8191, 100003):
        arrs = [formats.f32_to_bf16(rng.normal(size=n).astype(np.float32)) for _ in range(4)]
        devs = [torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(G.DEV) for a in arrs]
        acc = tq.discrepancy_stats(*devs).cpu().numpy()
        sb, sf, cnt = ofp4.discrepancy_stats(*arrs)
        assert acc[2] == cnt and abs(acc[0] - sb) <= 1e-6 * sb and abs(acc[1] - sf) <= 1e-6 * sf


def test_outputs_deterministic():
    G.say("determinism")
    xt, xr = _pair(256, 2048, 21)
    t, r = G.to_dev(xt, 256, 2048), G.to_dev(xr, 256, 2048)
    outs = []
    for _ in range(2):
        g = tq.encode_guidance(r, NV, 1, with_y=True)
        y, c = tq.guided_fake_quant(t, g, with_codes=True)
        outs.append([G.u8(g.guide), G.u8(g.scales), G.bits_of(g.y), G.bits_of(y), G.u8(c)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_writes_stay_in_bounds():
    """Canary bytes around every output survive each call."""
    G.say("canaries")
    rows, cols = 37, 2048
    xt, xr = _pair(rows, cols, 31)
    t, r = G.to_dev(xt, rows, cols), G.to_dev(xr, rows, cols)
    n = rows * cols
    PAD = 4096

    def guarded(nbytes, dtype=torch.uint8):
        raw = torch.full((nbytes + 2 * PAD,), 0xA5, dtype=torch.uint8, device=G.DEV)
        return raw, raw[PAD:PAD + nbytes].view(dtype)

    def intact(raw, nbytes):
        h = raw.cpu().numpy()
        return bool((h[:PAD] == 0xA5).all() and (h[PAD + nbytes:] == 0xA5).all())

    for fmt in (NV, MX):
        B = 16 if fmt == NV else 32
        rc, codes = guarded(n // 2)
        rs, scales = guarded(n // B)
        ry, yb = guarded(2 * n)
        rg, gs = guarded(8)
        tq.quantize_rtn(t, fmt, codes=codes.view(rows, cols // 2), scales=scales.view(rows, cols // B),
                        gscale_out=gs.view(torch.float32).view(1, 2) if fmt == NV else None,
                        y=yb.view(torch.bfloat16).view(rows, cols))
        torch.cuda.synchronize()
        assert intact(rc, n // 2) and intact(rs, n // B) and intact(ry, 2 * n) and intact(rg, 8)
        rb, bits = guarded(n // 8)
        g = tq.encode_guidance(r, fmt, 1, guide=bits.view(rows, cols // 8))
        ry2, y2 = guarded(2 * n)
        rc2, c2 = guarded(n // 2)
        tq.guided_fake_quant(t, g, with_codes=True, y=y2.view(torch.bfloat16).view(rows, cols),
                             codes=c2.view(rows, cols // 2))
        rr, refc = guarded(n // 2)
        tq.decode_guidance(t, g, ref_codes=refc.view(rows, cols // 2))
        torch.cuda.synchronize()
        assert intact(rb, n // 8) and intact(ry2, 2 * n) and intact(rc2, n // 2) and intact(rr, n // 2)


# ---------------------------------------------------------------- grouped calls

def _grouped_pair(G_, group_rows, cols, seed, mx=False):
    """G_ groups with different magnitudes, so every group has its own S."""
    xs, rs = [], []
    for g in range(G_):
        if mx:
            xt, xr = syn.mxfp4_pair(rows=group_rows, cols=cols, frac=0.01)
        else:
            xt, xr = syn.activation_pair(group_rows, cols, (91, seed, g))
        k = float(2.0 ** (3 * (g % 8) - 4)) * (1.0 + 0.37 * (g % 5))
        xs.append((xt.float() * k).to(torch.bfloat16))
        rs.append((xr.float() * k).to(torch.bfloat16))
    return syn.bits_u16(torch.cat(xs)).reshape(-1), syn.bits_u16(torch.cat(rs)).reshape(-1)


# (groups, group_rows, cols). Packed (NVFP4 groups of 2..1024 units, a power of
# two, several to a tile): (5, 2, 64), (300, 1, 2048) per-token rows with a
# ragged last tile, (1000, 1, 256) KV rows, (9, 4, 16), (5, 2, 4096).
GROUPED = [(3, 37, 2048), (5, 2, 64), (4, 64, 256), (2, 8192 // 32, 2048), (300, 1, 2048),
           (1000, 1, 256), (9, 4, 16), (5, 2, 4096)]
# MXFP4 blocks are 32 elements wide, so its cases need cols % 32 == 0 (the
# ABI rejects the rest; tests/test_abi_cpu.py covers that error).
GROUPED_CASES = [(f,) + c for f in (NV, MX) for c in GROUPED if f == NV or c[2] % 32 == 0]


@pytest.mark.parametrize("fmt,G_,gr,cols", GROUPED_CASES)
def test_grouped_quantize_and_encode(fmt, G_, gr, cols):
    G.say(f"grouped quantize/encode fmt={fmt} groups={G_} x ({gr},{cols})")
    xt, xr = _grouped_pair(G_, gr, cols, 1, mx=(fmt == MX))
    rows = G_ * gr
    G.check_quantize(xt, rows, cols, fmt, group_rows=gr)
    for bits in (1, 2, 3, 4):
        G.check_encode(xr, rows, cols, fmt, bits, group_rows=gr)
    if fmt == NV:
        G.check_quantize(xt, rows, cols, fmt, gscale=np.float32(0.75), group_rows=gr)


@pytest.mark.parametrize("fmt,G_,gr,cols", GROUPED_CASES)
def test_grouped_guided_and_decode(fmt, G_, gr, cols):
    G.say(f"grouped guided/decode fmt={fmt} groups={G_} x ({gr},{cols})")
    xt, xr = _grouped_pair(G_, gr, cols, 2, mx=(fmt == MX))
    rows = G_ * gr
    for bits in (0, 1, 2, 3, 4):
        G.check_guided(xt, xr, rows, cols, fmt, bits, group_rows=gr)
    for bits in (1, 2, 3):
        G.check_decode(xt, xr, rows, cols, fmt, group_rows=gr, bits=bits)


# ---------------------------------------------------------------- fused statistics

@pytest.mark.parametrize("fmt", [NV, MX])
@pytest.mark.parametrize("bits", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 2048), (256, 2048), (333, 256)])
def test_guided_fake_quant_stats(fmt, bits, rows, cols):
    G.say(f"guided_fake_quant_stats fmt={fmt} bits={bits} shape=({rows},{cols})")
    xt, xr = _pair(rows, cols, rows + 4, mx=(fmt == MX))
    G.check_guided_stats(xt, xr, rows, cols, fmt, bits)


@pytest.mark.parametrize("fmt", [NV, MX])
@pytest.mark.parametrize("bits", [0, 1, 2, 4])
@pytest.mark.parametrize("shift", [0, 1, 3])
def test_guided_wave_runs_unaligned_and_ragged(fmt, bits, shift):
    """The fused pass with no record or a 1-bit one reads a wave's scale and
    record bytes as dwords when the wave's run lies inside its group and
    starts on a dword, and per unit otherwise. NVFP4 groups of 37 rows x 2064
    columns (9,546 units) start off a dword in both planes and end in a
    ragged run (MXFP4, whose groups form one tensor: 111 x 2080); the planes
    are also moved to byte offsets 1 and 3. The plain pass, wider records and
    Reconstruct (per-unit reads) on the same inputs. GPU vs oracle."""
    G.say(f"guided wave runs fmt={fmt} bits={bits} shift={shift}")
    G_, gr = 3, 37
    cols = 2064 if fmt == NV else 2080
    xt, xr = _grouped_pair(G_, gr, cols, 5, mx=(fmt == MX))
    rows = G_ * gr
    rec_bits = 4 if bits == 0 else bits
    t, r = G.to_dev(xt, rows, cols), G.to_dev(xr, rows, cols)
    g = tq.encode_guidance(r, fmt, rec_bits, group_rows=gr)

    def moved(p, step):
        raw = torch.zeros(p.numel() + 64, dtype=torch.uint8, device=G.DEV)
        v = raw[step:step + p.numel()].view(p.shape)
        v.copy_(p)
        return v

    # records of 2 and 4 bits keep their 2- and 4-byte alignment
    g = g._replace(scales=moved(g.scales, shift), guide=moved(g.guide, shift * {1: 1, 2: 2, 4: 4}[rec_bits]))
    y, codes = tq.guided_fake_quant(t, g, bits=bits, with_codes=True)
    y2, codes2, acc = tq.guided_fake_quant_stats(t, r, g, bits=bits, with_codes=True)
    o_enc = G.oracle_encode(fmt, rec_bits, xr, rows, gr)
    o = G.oracle_guided(fmt, bits, xt, o_enc, rows, gr)
    what = f"fmt={fmt} bits={bits} shift={shift}"
    G.assert_same(G.bits_of(y), o["y"], f"guided y {what}")
    G.assert_same(G.u8(codes), o["codes"], f"guided codes {what}")
    G.assert_same(G.bits_of(y2), o["y"], f"guided y (stats) {what}")
    G.assert_same(G.u8(codes2), o["codes"], f"guided codes (stats) {what}")
    sb, sf, n = ofp4.discrepancy_stats(xt, xr, o["y"], o_enc["y"])
    a = acc.cpu().numpy()
    assert a[2] == n and G.rel_close(a[0], sb) and G.rel_close(a[1], sf), (a, sb, sf, n)
    if bits in (1, 2):
        ref = tq.decode_guidance(t, g)
        G.assert_same(G.u8(ref), G.oracle_decode(fmt, xt, o_enc, rows, gr, bits), f"reference codes {what}")


@pytest.mark.parametrize("fmt", [NV, MX])
def test_guided_fake_quant_stats_grouped_and_accumulated(fmt):
    G.say(f"guided_fake_quant_stats grouped fmt={fmt}")
    xt, xr = _grouped_pair(3, 37, 2048, 3, mx=(fmt == MX))
    a, _ = G.check_guided_stats(xt, xr, 111, 2048, fmt, 1, group_rows=37)
    # accumulate=True over two calls equals the sums of the two halves
    t, r = G.to_dev(xt, 111, 2048), G.to_dev(xr, 111, 2048)
    g = tq.encode_guidance(r, fmt, 1, group_rows=37)
    _, _, acc, cnt = tq.guided_fake_quant_stats(t, r, g, mismatch=True)
    one = cnt.clone()
    tq.guided_fake_quant_stats(t, r, g, acc=acc, accumulate=True, counts=cnt)
    b = acc.cpu().numpy()
    assert b[2] == 2 * a[2] and G.rel_close(b[0], 2 * a[0], 1e-12) and G.rel_close(b[1], 2 * a[1], 1e-12)
    assert torch.equal(cnt, 2 * one)
    # counts with accumulate=False overwrite whatever the tensor held
    cnt.fill_(-12345)
    tq.guided_fake_quant_stats(t, r, g, counts=cnt)
    assert torch.equal(cnt, one)


@pytest.mark.parametrize("fmt", [NV, MX])
def test_mismatch_counts_planted(fmt):
    """Rollout = training with 4000 elements scaled by 1.5, so that both
    histograms have entries beyond distance 1; each record width against the
    oracle. With the full-code record (bits=4) the guided code is the bracket
    end nearer the rollout code, so its total distance never exceeds RTN's."""
    G.say(f"mismatch counts, planted differences fmt={fmt}")
    xt, _ = _pair(64, 2048, 11, mx=(fmt == MX))
    xt = xt.reshape(-1)
    xr = xt.copy()
    rng = np.random.default_rng(5)
    idx = rng.choice(xt.size, 4000, replace=False)
    f = ofp4.bf16_to_f32(xr[idx]).astype(np.float32) * np.float32(1.5)
    xr[idx] = formats.f32_to_bf16(f)
    for bits in (4, 3, 2, 1, 0):
        G.check_guided_stats(xt, xr, 64, 2048, fmt, bits)
    t, r = G.to_dev(xt, 64, 2048), G.to_dev(xr, 64, 2048)
    *_, cnt = tq.guided_fake_quant_stats(t, r, tq.encode_guidance(r, fmt, 4), mismatch=True)
    c = cnt.cpu().numpy()
    d = np.arange(tq.MISMATCH_BINS)
    assert c[:15].sum() == c[15:30].sum() == xt.size
    assert (c[16:30] > 0).sum() >= 2                      # RTN: distances beyond 1 occur
    assert (d * c[:15]).sum() <= (d * c[15:30]).sum()
    assert (d * c[:15]).sum() < (d * c[15:30]).sum() or c[30] + c[31] == 0


@pytest.mark.parametrize("fmt", [NV, MX])
def test_guided_fake_quant_stats_extreme_values(fmt):
    """Squares that overflow binary32 and differences that underflow it take
    the exact binary64 path; corner-case scales as in the quantization test."""
    G.say(f"guided_fake_quant_stats extreme values fmt={fmt}")
    b = _edge_tensor()
    b2 = b.copy()
    b2[::3] ^= 0x0001
    b2[1::7] ^= 0x8000                       # sign flips: (x_t - x_r)^2 ~ (2x)^2 overflows binary32
    for bits in (0, 1, 2, 3, 4):
        G.check_guided_stats(b2, b, 16, 64, fmt, bits)
    tiny = np.zeros(64, np.uint16)
    tiny[:32] = np.arange(1, 33)             # bf16 subnormals: squares underflow binary32
    tiny2 = tiny.copy()
    tiny2[:32] += 1
    G.check_guided_stats(tiny2, tiny, 2, 32, fmt, 1)


def test_discrepancy_stats_extreme_values():
    G.say("discrepancy_stats extreme values")
    big = formats.f32_to_bf16(np.array([3e38, -3e38, 1e20, -1e-30, 0, 5] * 8, np.float32))
    tiny = np.arange(1, 49, dtype=np.uint16)
    for a, b in ((big, big[::-1].copy()), (tiny, tiny[::-1].copy())):
        devs = [torch.from_numpy(v.view(np.int16).copy()).view(torch.bfloat16).to(G.DEV) for v in (a, b, b, a)]
        acc = tq.discrepancy_stats(*devs).cpu().numpy()
        sb, sf, n = ofp4.discrepancy_stats(a, b, b, a)
        assert acc[2] == n and G.rel_close(acc[0], sb) and G.rel_close(acc[1], sf), (acc, sb, sf)


# ---------------------------------------------------------------- encode schedules

@pytest.fixture
def one_batch():
    """One amax pass over every group, then one quantize pass."""
    lib = tq.load()
    prev = lib.trace_set_encode_batch(1 << 40)
    yield
    lib.trace_set_encode_batch(prev)


@pytest.mark.parametrize("per_batch", [1, 2, 3, 1 << 40])
def test_encode_batches_grouped(per_batch):
    """Batches of 1, 2, 3 and all of 5 groups: every launch quantizes one
    batch and runs the amax pass of the next."""
    G.say(f"encode batches of {per_batch} groups, 5 groups x (37, 2048)")
    lib = tq.load()
    prev = lib.trace_set_encode_batch(per_batch)
    try:
        xt, xr = _grouped_pair(5, 37, 2048, 6)
        G.check_quantize(xt, 185, 2048, NV, group_rows=37)
        for bits in (1, 4):
            G.check_encode(xr, 185, 2048, NV, bits, group_rows=37)
        G.check_guided_stats(xt, xr, 185, 2048, NV, 1, group_rows=37)
    finally:
        lib.trace_set_encode_batch(prev)


def test_one_batch_corner_cases(one_batch):
    G.say("one-batch encode: scale corner cases and enumeration anchors")
    b = _edge_tensor()
    G.check_quantize(b, 16, 64, NV)
    G.check_encode(b, 16, 64, NV, 1)
    test_enumerate_bf16_block_max()


def test_schedules_agree_on_streamed_chunks():
    """The single-pass encode (the default for chunks of 8192 x 2048) and the
    two-pass schedule give identical encodings of 17 streamed chunks."""
    G.say("single pass vs two passes on [17 x 8192, 2048]")
    CH = syn.STREAM_CHUNK
    xr = torch.cat([syn.stream_pair(21, c, G.DEV)[1] for c in range(17)])
    lib = tq.load()
    outs = []
    for per_batch in (0, 1 << 40):
        prev = lib.trace_set_encode_batch(per_batch)
        try:
            g = tq.encode_guidance(xr, NV, 1, with_y=True, group_rows=CH)
            q = tq.quantize_rtn(xr, NV, group_rows=CH, with_y=False)
            torch.cuda.synchronize()
        finally:
            lib.trace_set_encode_batch(prev)
        outs.append([G.u8(g.guide), G.u8(g.scales), G.f32(g.gscale), G.bits_of(g.y), G.u8(q.codes)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("G_,gr,cols", [(2, 256, 2048), (17, 64, 2048), (3, 37, 2048), (2, 1024, 2048),
                                         (24, 1024, 2048)])
def test_single_pass_encode_waits_never_time_out(G_, gr, cols):
    """The device's count of the single-pass encode's bounded waits that gave
    up stays unchanged (every workgroup was resident), and the result is the
    oracle's."""
    G.say(f"single-pass encode wait counter, {G_} groups x ({gr},{cols})")
    xt, xr = _grouped_pair(G_, gr, cols, 8)
    rows = G_ * gr
    x = G.to_dev(xr, rows, cols)
    work = tq.quant_workspace(NV, rows, cols, gr, device=G.DEV)
    fails0 = tq.encode_wait_failures()
    g = tq.encode_guidance(x, NV, 1, with_y=True, group_rows=gr, work=work)
    torch.cuda.synchronize()
    words = work.view(torch.int32).cpu().numpy()
    assert tq.encode_wait_failures() == fails0
    # only the single pass publishes S (16 copies, 64 words apart, per group)
    S_bits = g.gscale.reshape(-1, 2)[:, 0].cpu().numpy().view(np.int32)
    pub = words[G_ * 1024:G_ * 2048].reshape(G_, 16, 64)[:, :, 0]
    assert np.array_equal(pub, np.repeat(S_bits[:, None], 16, axis=1)), "single pass not used"
    o = G.oracle_encode(NV, 1, xr, rows, gr)
    G.assert_same(G.u8(g.guide), o["guide"], "guide")
    G.assert_same(G.bits_of(g.y), o["y"], "rollout y")
    G.assert_same(G.f32(g.gscale).reshape(-1, 2)[:, 0], o["gscale"], "S")


def _encode_schedule_check(G_, gr, cols, bits, seed, single):
    """encode_guidance with one S per group against the oracle; `single`
    says whether the single-pass encode must have run (it alone publishes S
    to the workspace's S words) or the two-pass one."""
    xt, xr = _grouped_pair(G_, gr, cols, seed)
    rows = G_ * gr
    x = G.to_dev(xr, rows, cols)
    work = tq.quant_workspace(NV, rows, cols, gr, device=G.DEV)
    work.zero_()
    fails0 = tq.encode_wait_failures()
    g = tq.encode_guidance(x, NV, bits, with_y=True, group_rows=gr, work=work)
    torch.cuda.synchronize()
    words = work.view(torch.int32).cpu().numpy()
    S_bits = g.gscale.reshape(-1, 2)[:, 0].cpu().numpy().view(np.int32)
    pub = words[G_ * 1024:G_ * 2048].reshape(G_, 16, 64)[:, :, 0]
    assert np.array_equal(pub, np.repeat(S_bits[:, None], 16, axis=1)) == single, "unexpected schedule"
    assert tq.encode_wait_failures() == fails0
    o = G.oracle_encode(NV, bits, xr, rows, gr)
    G.assert_same(G.u8(g.guide), o["guide"], "guide")
    G.assert_same(G.bits_of(g.y), o["y"], "rollout y")
    G.assert_same(G.u8(g.scales), o["scales"], "scales")
    G.assert_same(G.f32(g.gscale).reshape(-1, 2)[:, 0], o["gscale"], "S")


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("G_,gr,cols", [(40, 37, 48), (1200, 3, 2048)])
def test_single_pass_tile_geometry(G_, gr, cols, bits):
    """Single-pass encodes whose tiles are not whole 64-unit multiples of the
    group (40 groups of 222 units: tiles of 64, 64, 64 and 30 units, 40 groups
    in flight) and whose workgroups take several groups in turn (1200 groups
    of 768 units, 511 in flight), for every plane width, with y."""
    G.say(f"single-pass tile geometry, {G_} groups x ({gr},{cols}), bits {bits}")
    _encode_schedule_check(G_, gr, cols, bits, 17 + bits, single=True)


def test_single_group_uses_two_passes():
    """A call of one group (one chunk, or one KV tensor) goes through the
    two-pass schedule, which is faster there; the results are the oracle's."""
    G.say("one group: two-pass schedule")
    _encode_schedule_check(1, 512, 2048, 1, 43, single=False)
    _encode_schedule_check(1, 4096, 256, 4, 44, single=False)


def test_single_pass_largest_group_and_the_next():
    """The largest group the single-pass encode holds on chip at once
    ((2 x CUs - 1) tiles of 4224 units) is encoded in one pass; a group a
    few rows larger falls back to two passes. Both match the oracle."""
    cus = torch.cuda.get_device_properties(G.DEV).multi_processor_count
    cols = 2048
    rows_max = (2 * cus - 1) * 4224 * 8 // cols
    G.say(f"single-pass boundary: groups of {rows_max} and {rows_max + 3} rows x {cols} ({cus} CUs)")
    _encode_schedule_check(2, rows_max, cols, 1, 41, single=True)
    _encode_schedule_check(2, rows_max + 3, cols, 1, 42, single=False)


def _random_cases(n, seed):
    """Seeded random shapes: format, [rows, cols], group rows (0 or a divisor
    of rows), record width, guided width (0 or the record's), with or without
    y. At most ~2M elements each, so the oracle keeps up."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        fmt = NV if rng.random() < 0.7 else MX
        cols = int(rng.choice([16, 32, 48, 64, 96, 128, 256, 512, 1024, 2048, 4096]))
        if fmt == MX and cols % 32:
            continue
        rows = int(rng.integers(1, min(4096, 2_000_000 // cols) + 1))
        divs = [d for d in range(1, rows + 1) if rows % d == 0]
        gr = 0 if rng.random() < 0.25 else int(rng.choice(divs))
        bits = int(rng.integers(1, 5))
        out.append((fmt, rows, cols, gr, bits, int(rng.choice([0, bits])), bool(rng.random() < 0.5),
                    int(rng.integers(1 << 30))))
    return out


def test_random_shapes():
    """40 seeded random shapes through encode_guidance and guided_fake_quant
    (single-pass, packed and two-pass schedules as the shapes fall), each
    group with its own magnitude, against the oracle."""
    for k, (fmt, rows, cols, gr, bits, gbits, with_y, seed) in enumerate(_random_cases(40, 2026)):
        G.say(f"random case {k}: fmt {fmt} [{rows}, {cols}] group_rows {gr} bits {bits}/{gbits} y {with_y}")
        xt, xr = syn.activation_pair(rows, cols, (97, seed))
        n_g = rows // gr if gr else 1
        mag = 2.0 ** np.random.default_rng(seed).integers(-8, 9, n_g).astype(np.float32)
        scale = torch.from_numpy(np.repeat(mag, rows // n_g)).reshape(-1, 1)
        xtb = syn.bits_u16((xt.float() * scale).to(torch.bfloat16)).reshape(-1)
        xrb = syn.bits_u16((xr.float() * scale).to(torch.bfloat16)).reshape(-1)
        G.check_encode(xrb, rows, cols, fmt, bits, with_y=with_y, group_rows=gr)
        G.check_guided(xtb, xrb, rows, cols, fmt, gbits, group_rows=gr)


def test_random_shapes_fused_pass():
    """24 seeded random shapes through guided_fake_quant_stats (with and
    without mismatch counts), records of 0 to 4 bits weighted to 0 and 1
    (whose waves read their scale and record bytes as dwords where a run is
    whole and aligned): group sizes, ragged runs and group starts as the
    shapes fall, each group with its own magnitude, against the oracle."""
    rng = np.random.default_rng(2027)
    done = 0
    while done < 24:
        fmt = NV if rng.random() < 0.7 else MX
        cols = int(rng.choice([16, 48, 64, 96, 208, 256, 1040, 2048, 2064]))
        if fmt == MX and cols % 32:
            continue
        rows = int(rng.integers(1, min(2048, 1_000_000 // cols) + 1))
        divs = [d for d in range(1, rows + 1) if rows % d == 0]
        gr = 0 if rng.random() < 0.3 else int(rng.choice(divs))
        bits = int(rng.choice([0, 1, 1, 0, 2, 4]))
        seed = int(rng.integers(1 << 30))
        G.say(f"random fused case {done}: fmt {fmt} [{rows}, {cols}] group_rows {gr} bits {bits}")
        xt, xr = syn.activation_pair(rows, cols, (98, seed))
        n_g = rows // gr if gr else 1
        mag = 2.0 ** np.random.default_rng(seed).integers(-8, 9, n_g).astype(np.float32)
        scale = torch.from_numpy(np.repeat(mag, rows // n_g)).reshape(-1, 1)
        xtb = syn.bits_u16((xt.float() * scale).to(torch.bfloat16)).reshape(-1)
        xrb = syn.bits_u16((xr.float() * scale).to(torch.bfloat16)).reshape(-1)
        G.check_guided_stats(xtb, xrb, rows, cols, fmt, bits, group_rows=gr)
        done += 1


# ---------------------------------------------------------------- row-offset groups

def _offset_groups_pair(sizes, cols, seed):
    """Consecutive groups of the given row counts (some empty), each with its
    own magnitude."""
    xs, rs = [], []
    for g, n in enumerate(sizes):
        if n == 0:
            continue
        xt, xr = syn.activation_pair(n, cols, (94, seed, g))
        k = float(2.0 ** (3 * (g % 7) - 6)) * (1.0 + 0.29 * (g % 3))
        xs.append((xt.float() * k).to(torch.bfloat16))
        rs.append((xr.float() * k).to(torch.bfloat16))
    return syn.bits_u16(torch.cat(xs)).reshape(-1), syn.bits_u16(torch.cat(rs)).reshape(-1)


def _oracle_offsets(fmt, bits, xt_b, xr_b, cols, offs):
    """The oracle per group: each group's rows as one tensor."""
    enc, gd, S = [], [], []
    for g in range(len(offs) - 1):
        r0, r1 = int(offs[g]), int(offs[g + 1])
        es = slice(r0 * cols, r1 * cols)
        if r1 == r0:
            S.append((1.0, 0.0))
            continue
        o = ofp4.encode_guidance(fmt, 4 if bits == 0 else bits, xr_b[es])
        og = ofp4.guided_fake_quant(fmt, bits, xt_b[es], None if bits == 0 else o["guide"], o["scales"],
                                    o["gscale"])
        enc.append(o)
        gd.append(og)
        S.append((o["gscale"], o["amax"]))
    cat = lambda parts, k: np.concatenate([p[k] for p in parts])  # noqa: E731
    return cat(enc, "guide"), cat(enc, "scales"), cat(enc, "y"), cat(gd, "y"), cat(gd, "codes"), S


@pytest.mark.parametrize("sizes,cols", [([0, 37, 1, 300, 0, 0, 512, 100, 50], 2048),
                                        ([3, 0, 64, 1, 9], 256), ([7], 64), ([0, 0, 5], 16)])
def test_row_offset_groups(sizes, cols):
    """encode_guidance_grouped / guided_fake_quant_grouped against the oracle
    run on each group's rows, every record width; empty groups get {1, 0}."""
    G.say(f"row-offset groups {sizes} x {cols}")
    _check_row_offset_groups(sizes, cols, (1, 2, 3, 4))


@pytest.mark.parametrize("n_groups", [3000, 9000])
def test_row_offset_many_groups(n_groups):
    """Thousands of small row-offset groups, a quarter of them empty. Up to
    4096 groups one kernel derives the offsets, tile starts and tile table
    (3000); beyond that the prep kernel and the table kernel, whose search
    runs in memory past 8192 groups (9000); both against the oracle."""
    sizes = np.random.default_rng(n_groups).integers(0, 4, n_groups).tolist()
    G.say(f"row-offset groups: {n_groups} groups of 0..3 rows x 16")
    _check_row_offset_groups(sizes, 16, (1,))


def _check_row_offset_groups(sizes, cols, widths):
    xt_b, xr_b = _offset_groups_pair(sizes, cols, len(sizes))
    rows = sum(sizes)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    doffs = torch.from_numpy(offs).to(G.DEV)
    xt, xr = G.to_dev(xt_b, rows, cols), G.to_dev(xr_b, rows, cols)
    for bits in widths:
        g = tq.encode_guidance_grouped(xr, doffs, NV, bits, with_y=True)
        guide, scales, yr, _, _, S = _oracle_offsets(NV, bits, xt_b, xr_b, cols, offs)
        G.assert_same(G.u8(g.guide), guide, f"guide bits={bits}")
        G.assert_same(G.u8(g.scales), scales, "scales")
        G.assert_same(G.bits_of(g.y), yr, "rollout y")
        gs = G.f32(g.gscale).reshape(-1, 2)
        G.assert_same(gs, np.array(S, np.float32), "{S, A} per group")
        for gb in (bits, 0):
            y, codes = tq.guided_fake_quant(xt, g, bits=gb, with_codes=True)
            _, _, _, yg, cg, _ = _oracle_offsets(NV, gb, xt_b, xr_b, cols, offs) if gb == 0 else \
                _oracle_offsets(NV, bits, xt_b, xr_b, cols, offs)
            G.assert_same(G.bits_of(y), yg, f"guided y bits={gb}")
            G.assert_same(G.u8(codes), cg, f"guided codes bits={gb}")


def _grouped_both_schedules(xr, doffs, bits, with_y):
    """encode_guidance_grouped in one pass (the default) and in two passes
    (forced by a batch size), plus the device's count of waits that gave up
    during the single pass."""
    lib = _abi.load()
    fails0 = tq.encode_wait_failures()
    one = tq.encode_guidance_grouped(xr, doffs, NV, bits, with_y=with_y)
    torch.cuda.synchronize()
    fails = tq.encode_wait_failures() - fails0
    prev = lib.trace_set_encode_batch(1)
    try:
        two = tq.encode_guidance_grouped(xr, doffs, NV, bits, with_y=with_y)
        torch.cuda.synchronize()
    finally:
        lib.trace_set_encode_batch(prev)
    return one, two, fails


@pytest.mark.parametrize("sizes,cols,bits", [
    ([0, 37, 1, 300, 0, 0, 512, 100, 50], 2048, 1),                 # small experts, some empty
    ([4096] * 16, 2048, 4),                                          # 16 experts of 4096 rows (2048 tiles each)
    ([100, 60000, 0, 5436], 2048, 1),                                # one expert with most rows: tiles read twice
    ([65536], 2048, 2),                                              # a single group larger than the grid holds
    ([1040, 2048, 2064, 1500, 16, 1100] * 3, 2048, 1),               # 65, 128, 129, 94, 1, 69 tiles: both sides of the
                                                                     # combining workgroup's small-group limit
    (np.random.default_rng(5).integers(0, 600, 256).tolist(), 2048, 1),   # a routed MoE layer's shape
])
def test_row_offset_single_pass_equals_two_passes(sizes, cols, bits):
    """The single-pass encode of row-offset groups (a device-built table of
    tiles, one pass over the input; groups larger than the resident grid
    holds have their tiles' maxima read first) against the two-pass schedule,
    bit for bit, every S against the oracle's scale of the exact amax, and
    sampled rows of the largest group against the oracle."""
    _single_vs_two_passes(sizes, cols, bits)


@pytest.mark.parametrize("extra", [1, 2])
def test_row_offset_single_pass_group_of_grid_size(extra):
    """A group of W + 1 tiles of 4096 units (W = tile workgroups of the
    launch, 2 per CU less the combining one): the largest group that is
    complete one round after its last tile, and W + 2, the smallest whose
    tiles' maxima are read first; between small groups, against the
    two-pass schedule and the oracle."""
    W = 2 * torch.cuda.get_device_properties(0).multi_processor_count - 1
    cols = 2048                              # 256 units per row: 16 rows per tile
    _single_vs_two_passes([40, (W + extra) * 16, 300, 0, 17], cols, 1)


@pytest.mark.parametrize("n_groups", [4096, 4097])
def test_row_offset_group_count_limit(n_groups):
    """Up to 4096 row-offset groups the encode takes one pass; one more group
    takes the two-pass schedule. Both against the oracle."""
    sizes = np.random.default_rng(n_groups + 1).integers(0, 4, n_groups).tolist()
    G.say(f"row-offset groups: {n_groups} groups of 0..3 rows x 16")
    _check_row_offset_groups(sizes, 16, (1,))


def test_row_offset_random_cases():
    """16 seeded random row-offset layouts (1 to 200 groups, runs of empty
    groups, one dominant group in some, widths 16 to 2048 columns, every
    record width): the default encode (one pass up to 4096 groups) against
    the two-pass schedule bit for bit, and both against the oracle run on
    each group's rows."""
    rng = np.random.default_rng(2027)
    for k in range(16):
        cols = int(rng.choice([16, 48, 128, 256, 2048]))
        n_groups = int(rng.integers(1, 201))
        cap = max(1, 1_500_000 // cols)                    # elements per case stay within ~1.5M
        sizes = rng.geometric(0.02, n_groups) - 1          # many small, some empty
        sizes[rng.random(n_groups) < 0.2] = 0
        if k % 4 == 3:
            sizes[int(rng.integers(0, n_groups))] += cap // 2   # one dominant group
        if sizes.sum() > cap:
            sizes = (sizes * (cap / sizes.sum())).astype(np.int64)
        sizes = [int(v) for v in sizes]
        if sum(sizes) == 0:
            sizes[0] = 1
        bits = int(rng.integers(1, 5))
        G.say(f"row-offset random case {k}: {n_groups} groups, {sum(sizes)} rows x {cols}, bits {bits}")
        xt_b, xr_b = _offset_groups_pair(sizes, cols, 600 + k)
        rows = sum(sizes)
        offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
        doffs = torch.from_numpy(offs).to(G.DEV)
        xr = G.to_dev(xr_b, rows, cols)
        one, two, fails = _grouped_both_schedules(xr, doffs, bits, True)
        assert fails == 0
        assert torch.equal(one.guide, two.guide) and torch.equal(one.scales, two.scales), k
        assert torch.equal(one.gscale, two.gscale), k
        assert torch.equal(one.y.view(torch.int16), two.y.view(torch.int16)), k
        guide, scales, yr, _, _, S = _oracle_offsets(NV, bits, xt_b, xr_b, cols, offs)
        G.assert_same(G.u8(one.guide), guide, f"case {k} guide")
        G.assert_same(G.u8(one.scales), scales, f"case {k} scales")
        G.assert_same(G.bits_of(one.y), yr, f"case {k} rollout y")
        G.assert_same(G.f32(one.gscale).reshape(-1, 2), np.array(S, np.float32), f"case {k} {{S, A}}")


def _single_vs_two_passes(sizes, cols, bits):
    sizes = [int(v) for v in sizes]
    rows = sum(sizes)
    G.say(f"row-offset single pass vs two passes: {len(sizes)} groups, {rows} rows x {cols}, bits {bits}")
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device=G.DEV)
    r0 = 0
    for g, n in enumerate(sizes):
        if n:
            _, xr = syn.activation_pair(n, cols, (95, len(sizes), g), G.DEV)
            x[r0:r0 + n] = (xr.float() * float(2.0 ** (g % 9 - 4))).to(torch.bfloat16)
        r0 += n
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    doffs = torch.from_numpy(offs).to(G.DEV)
    one, two, fails = _grouped_both_schedules(x, doffs, bits, True)
    assert fails == 0
    assert torch.equal(one.guide, two.guide) and torch.equal(one.scales, two.scales)
    assert torch.equal(one.gscale, two.gscale)
    assert torch.equal(one.y.view(torch.int16), two.y.view(torch.int16))
    amax = (x.view(torch.int16) & 0x7FFF).amax(dim=1).cpu().numpy().astype(np.uint16)
    gs = G.f32(one.gscale).reshape(-1, 2)
    for g in range(len(sizes)):
        a0, a1 = int(offs[g]), int(offs[g + 1])
        A = ofp4.bf16_to_f32(amax[a0:a1]).max() if a1 > a0 else np.float32(0)
        assert gs[g, 1] == A and gs[g, 0] == ofp4.nvfp4_global_scale(A), g
    big = int(np.argmax(sizes))
    a0 = int(offs[big])
    S = gs[big, 0]
    xb = G.bits_of(x[a0:a0 + min(64, sizes[big])])
    o = ofp4.encode_guidance(NV, bits, xb, S)
    n0, n1 = a0 * cols, (a0 + xb.size // cols) * cols
    G.assert_same(G.u8(one.guide).reshape(-1)[n0 * bits // 8:n1 * bits // 8], o["guide"], "largest group guide")
    G.assert_same(G.u8(one.scales).reshape(-1)[n0 // 16:n1 // 16], o["scales"], "largest group scales")
    G.assert_same(G.bits_of(one.y)[n0:n1], o["y"], "largest group y")


def test_row_offset_groups_bad_offsets_and_uncovered_rows():
    """Offsets outside [0, rows] or decreasing are clamped and made
    nondecreasing; rows outside [off[0], off[G]) are left untouched."""
    G.say("row-offset groups: bad offsets, canaries")
    cols, rows = 256, 40
    xt_b, xr_b = _offset_groups_pair([rows], cols, 3)
    xr = G.to_dev(xr_b, rows, cols)
    bad = np.array([5, -3, 20, 12, 33, 90], np.int64)          # -> 5 5 20 20 33 40
    eff = np.maximum.accumulate(np.clip(bad, 0, rows))
    doffs = torch.from_numpy(bad).to(G.DEV)
    guide = torch.full((rows, cols // 8), 0xA5, dtype=torch.uint8, device=G.DEV)
    y = torch.full((rows, cols), 0x1234, dtype=torch.int16, device=G.DEV).view(torch.bfloat16)
    g = tq.encode_guidance_grouped(xr, doffs, NV, 1, with_y=True, guide=guide, y=y)
    torch.cuda.synchronize()
    gu, yy = G.u8(g.guide).reshape(rows, -1), G.bits_of(g.y).reshape(rows, -1)
    assert (gu[:5] == 0xA5).all() and (yy[:5] == 0x1234).all()      # rows before off[0]
    for k in range(len(eff) - 1):
        r0, r1 = int(eff[k]), int(eff[k + 1])
        if r1 == r0:
            assert tuple(G.f32(g.gscale).reshape(-1, 2)[k]) == (1.0, 0.0)
            continue
        o = ofp4.encode_guidance(NV, 1, xr_b[r0 * cols:r1 * cols])
        G.assert_same(gu[r0:r1].reshape(-1), o["guide"], f"group {k} guide")
        G.assert_same(yy[r0:r1].reshape(-1), o["y"], f"group {k} y")


def test_row_offset_groups_mxfp4_equals_ungrouped():
    G.say("row-offset groups, MXFP4")
    xt_b, xr_b = _offset_groups_pair([10, 0, 22], 2048, 5)
    xt, xr = G.to_dev(xt_b, 32, 2048), G.to_dev(xr_b, 32, 2048)
    doffs = torch.tensor([0, 10, 10, 32], dtype=torch.int64, device=G.DEV)
    g1 = tq.encode_guidance_grouped(xr, doffs, MX, 1, with_y=True)
    g0 = tq.encode_guidance(xr, MX, 1, with_y=True)
    assert g1.gscale is None
    assert torch.equal(g1.guide, g0.guide) and torch.equal(g1.scales, g0.scales)
    y1, _ = tq.guided_fake_quant(xt, g1)
    y0, _ = tq.guided_fake_quant(xt, g0)
    assert torch.equal(y1.view(torch.int16), y0.view(torch.int16))
