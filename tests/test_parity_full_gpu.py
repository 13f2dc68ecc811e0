"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (one call per tensor or per streamed layer).

The oracle is too slow for whole tensors, so every block-level output is
checked on sampled row ranges: the oracle quantizes those rows with the
group's global scale (computed by the oracle from the whole group's amax),
which fixes every block exactly. Properties that hold at any size are checked
on everything: the group scales against the oracle's amax, duplicate routed
rows giving identical outputs, the fused statistics against the oracle's SB
and against sums over the library's own (sample-verified) outputs.
"""

import numpy as np
import pytest
import torch

import precision_rl_nvfp4_amd as tq
import synthetic as syn
from oracle import fp4 as ofp4
from tests import _gpu as G

pytestmark = pytest.mark.gpu

NV, MX = tq.NVFP4, tq.MXFP4


def _bits(t):
    return G.bits_of(t)


def _samples(rows, k=3, span=48):
    """k row ranges spread over the tensor (first, middle, last), `span` rows each."""
    starts = sorted({0, max(0, rows // 2 - span // 2), max(0, rows - span)})[:k]
    return [(s, min(rows, s + span)) for s in starts]


def _group_S(fmt, xb_group):
    if fmt != NV:
        return None
    return ofp4.nvfp4_global_scale(ofp4.tensor_amax(xb_group))


def _check_rows(fmt, bits, xt_b, xr_b, cols, r0, r1, S, enc, y_g=None, codes_g=None, y_r=None,
                gbits=None):
    """Oracle on rows [r0, r1) of one group against the library's planes: the
    oracle encodes the rollout rows with the group scale S (the oracle's own)
    and guides the training rows with its own record (gbits: guided bits,
    default the record's)."""
    B = ofp4.BLOCK[fmt]
    es = slice(r0 * cols, r1 * cols)
    o = ofp4.encode_guidance(fmt, bits, xr_b[es], S)
    G.assert_same(G.u8(enc.guide).reshape(-1)[r0 * cols * bits // 8:r1 * cols * bits // 8], o["guide"],
                  f"guide rows {r0}:{r1}")
    G.assert_same(G.u8(enc.scales).reshape(-1)[r0 * cols // B:r1 * cols // B], o["scales"],
                  f"scales rows {r0}:{r1}")
    if y_r is not None:
        G.assert_same(_bits(y_r)[es], o["y"], f"rollout y rows {r0}:{r1}")
    if y_g is not None:
        gb = bits if gbits is None else gbits
        og = ofp4.guided_fake_quant(fmt, gb, xt_b[es], None if gb == 0 else o["guide"], o["scales"], S)
        G.assert_same(_bits(y_g)[es], og["y"], f"guided y rows {r0}:{r1}")
        if codes_g is not None:
            G.assert_same(G.u8(codes_g).reshape(-1)[r0 * cols // 2:r1 * cols // 2], og["codes"],
                          f"guided codes rows {r0}:{r1}")
    return o


def test_stream_layer_bench_configuration():
    """One streamed layer exactly as the benchmark calls it: 17 chunks of
    [8192, 2048] in one call, one global scale per chunk; encode (bits=1),
    then guided_fake_quant_stats (bits=1)."""
    G.say("full size: streamed layer, 17 x [8192, 2048], group_rows=8192")
    layer, chunks, CH = 20, 17, syn.STREAM_CHUNK
    dev = G.DEV
    sigma = syn.stream_sigma(layer, dev)
    xt = torch.empty((chunks * CH, syn.HIDDEN), dtype=torch.bfloat16, device=dev)
    xr = torch.empty_like(xt)
    for c in range(chunks):
        a, b = syn.stream_pair(layer, c, dev, sigma=sigma)
        xt[c * CH:(c + 1) * CH].copy_(a)
        xr[c * CH:(c + 1) * CH].copy_(b)
    work = tq.quant_workspace(NV, chunks * CH, syn.HIDDEN, CH, device=dev)
    fails0 = tq.encode_wait_failures()
    g = tq.encode_guidance(xr, NV, 1, with_y=True, group_rows=CH, work=work)
    y, codes, acc, counts = tq.guided_fake_quant_stats(xt, xr, g, with_codes=True, mismatch=True)
    y_plain, _ = tq.guided_fake_quant(xt, g)
    torch.cuda.synchronize()
    # no bounded wait of the single-pass encode gave up
    assert tq.encode_wait_failures() == fails0
    assert torch.equal(y.view(torch.int16), y_plain.view(torch.int16))
    # mismatch counts: the oracle's count over the whole code planes (rollout
    # codes from a full-code record, RTN codes under the rollout scales), whose
    # codes the row samples below pin to the oracle
    g4 = tq.encode_guidance(xr, NV, 4, group_rows=CH)
    y_rtn, codes_rtn = tq.guided_fake_quant(xt, g, bits=0, with_codes=True)
    want = G.oracle_plane_counts(codes, g4.guide, codes_rtn)
    G.assert_same(counts.cpu().numpy(), want, "mismatch counts, streamed layer")
    assert want[:15].sum() == xt.numel()
    G.say("  mismatch counts equal the oracle's")
    xt_b, xr_b = _bits(xt), _bits(xr)
    gs = G.f32(g.gscale).reshape(chunks, 2)
    n_chunk = CH * syn.HIDDEN
    sb_total = 0.0
    S_oracle = []
    for c in range(chunks):
        es = slice(c * n_chunk, (c + 1) * n_chunk)
        A = ofp4.tensor_amax(xr_b[es])
        S_oracle.append(ofp4.nvfp4_global_scale(A))
        assert gs[c, 1] == A and gs[c, 0] == S_oracle[c], (c, gs[c])
        d = (ofp4.bf16_to_f32(xt_b[es]).astype(np.float64) - ofp4.bf16_to_f32(xr_b[es]).astype(np.float64))
        sb_total += float(np.sum(d * d))
    for c in (0, 8, 16):
        for r0, r1 in _samples(CH):
            rr0, rr1 = c * CH + r0, c * CH + r1
            _check_rows(NV, 1, xt_b, xr_b, syn.HIDDEN, rr0, rr1, S_oracle[c], g, y_g=y, codes_g=codes,
                        y_r=g.y)
            _check_rows(NV, 4, xt_b, xr_b, syn.HIDDEN, rr0, rr1, S_oracle[c], g4)
            _check_rows(NV, 1, xt_b, xr_b, syn.HIDDEN, rr0, rr1, S_oracle[c], g, y_g=y_rtn,
                        codes_g=codes_rtn, gbits=0)
    # vanilla fake quantization of X_t with its own chunk scales (codes, y) and
    # the 1-bit Reconstruct alone, as the benchmark times them per layer
    q = tq.quantize_rtn(xt, NV, group_rows=CH, with_y=True)
    ref = tq.decode_guidance(xt, g)
    torch.cuda.synchronize()
    qs = G.f32(q.gscale).reshape(chunks, 2)
    cols = syn.HIDDEN
    for c in (0, 16):
        es = slice(c * n_chunk, (c + 1) * n_chunk)
        St = ofp4.nvfp4_global_scale(ofp4.tensor_amax(xt_b[es]))
        assert qs[c, 0] == St, (c, qs[c])
        for r0, r1 in _samples(CH, span=32):
            rr0, rr1 = c * CH + r0, c * CH + r1
            e2 = slice(rr0 * cols, rr1 * cols)
            oq = ofp4.quantize_rtn(NV, xt_b[e2], St)
            G.assert_same(G.u8(q.codes).reshape(-1)[rr0 * cols // 2:rr1 * cols // 2], oq["codes"],
                          f"rtn codes chunk {c} rows {r0}:{r1}")
            G.assert_same(_bits(q.y)[e2], oq["y"], f"rtn y chunk {c} rows {r0}:{r1}")
            o_enc = ofp4.encode_guidance(NV, 1, xr_b[e2], S_oracle[c])
            od = ofp4.decode_guidance(NV, xt_b[e2], o_enc["guide"], o_enc["scales"], S_oracle[c], bits=1)
            G.assert_same(G.u8(ref).reshape(-1)[rr0 * cols // 2:rr1 * cols // 2], od,
                          f"decode chunk {c} rows {r0}:{r1}")
    a = acc.cpu().numpy()
    assert a[2] == xt.numel()
    assert G.rel_close(a[0], sb_total), (a[0], sb_total)
    # SF: the oracle's sums over the guided and rollout outputs (sample-verified above)
    sb, sf, n = G.oracle_plane_sums(xt, xr, y, g.y)
    assert a[2] == n and G.rel_close(a[0], sb) and G.rel_close(a[1], sf), (a, (sb, sf, n))


@pytest.mark.parametrize("rows", [32764, 32768, 32772])
def test_guided_stats_reduction_split_boundary(rows):
    """guided_fake_quant_stats reduces its per-tile sums in one workgroup
    below 8,192 tiles and in eight from there (each a fixed slice, the last to
    finish adding the eight in order): 8,191, 8,192 and 8,193 tiles of 1024
    units over [rows, 2048] with one global scale. SB and SF against the
    oracle's float64 sums over the inputs and the (row-sampled) outputs; with
    accumulate=True a second call adds the same sums; the result is the same
    bits on a repeat."""
    G.say(f"full size: stats reduction at the split boundary, rows={rows}")
    dev = G.DEV
    CH = syn.STREAM_CHUNK
    sigma = syn.stream_sigma(3, dev)
    xt = torch.empty((4 * CH + CH, syn.HIDDEN), dtype=torch.bfloat16, device=dev)
    xr = torch.empty_like(xt)
    for c in range(5):
        a, b = syn.stream_pair(3, c, dev, sigma=sigma)
        xt[c * CH:(c + 1) * CH].copy_(a)
        xr[c * CH:(c + 1) * CH].copy_(b)
        del a, b
    xt, xr = xt[:rows].contiguous(), xr[:rows].contiguous()
    g = tq.encode_guidance(xr, NV, 1, with_y=True)
    y, codes, acc = tq.guided_fake_quant_stats(xt, xr, g, with_codes=True)
    _, _, acc_again = tq.guided_fake_quant_stats(xt, xr, g)
    tq.guided_fake_quant_stats(xt, xr, g, acc=acc_again, accumulate=True)
    torch.cuda.synchronize()
    xt_b, xr_b = _bits(xt), _bits(xr)
    S = _group_S(NV, xr_b)
    for r0, r1 in _samples(rows):
        _check_rows(NV, 1, xt_b, xr_b, syn.HIDDEN, r0, r1, S, g, y_g=y, codes_g=codes, y_r=g.y)
    a = acc.cpu().numpy()
    sb, sf, n = G.oracle_plane_sums(xt, xr, y, g.y)
    assert a[2] == n == rows * syn.HIDDEN and G.rel_close(a[0], sb) and G.rel_close(a[1], sf), (a, (sb, sf, n))
    b = acc_again.cpu().numpy()
    assert b[2] == 2 * a[2] and b[0] == 2 * a[0] and b[1] == 2 * a[1], (a, b)


def test_guided_stats_two_layers_in_one_call():
    """guided_fake_quant_stats over two streamed layers in one call (34
    chunks of [8192, 2048]: 69,632 tiles of 1024 units, past the 65,536 that
    one reduction workgroup sums, so the per-tile sums go through the
    two-level reduction). SB and SF against the oracle's float64 sums over the inputs
    and the (row-sampled) outputs; the same sums from the two per-layer calls,
    which take the one-level reduction."""
    G.say("full size: guided_fake_quant_stats over 2 streamed layers in one call")
    chunks, CH = 17, syn.STREAM_CHUNK
    dev = G.DEV
    xt = torch.empty((2 * chunks * CH, syn.HIDDEN), dtype=torch.bfloat16, device=dev)
    xr = torch.empty_like(xt)
    for li, layer in enumerate((20, 21)):
        sigma = syn.stream_sigma(layer, dev)
        for c in range(chunks):
            a, b = syn.stream_pair(layer, c, dev, sigma=sigma)
            r0 = (li * chunks + c) * CH
            xt[r0:r0 + CH].copy_(a)
            xr[r0:r0 + CH].copy_(b)
            del a, b
    rows = xt.shape[0]
    assert rows * syn.HIDDEN // 16384 > 32768
    g = tq.encode_guidance(xr, NV, 1, with_y=True, group_rows=CH)
    y, _, acc = tq.guided_fake_quant_stats(xt, xr, g)
    half = rows // 2
    gl = [tq.Guidance(NV, 1, g.guide[s], g.scales[s], g.gscale[k], None, CH)
          for s, k in ((slice(0, half), slice(0, chunks)), (slice(half, rows), slice(chunks, 2 * chunks)))]
    acc_l = torch.zeros(3, dtype=torch.float64, device=dev)
    y_l = torch.empty_like(y)
    tq.guided_fake_quant_stats(xt[:half], xr[:half], gl[0], acc=acc_l, y=y_l[:half])
    tq.guided_fake_quant_stats(xt[half:], xr[half:], gl[1], acc=acc_l, accumulate=True, y=y_l[half:])
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_l.view(torch.int16))
    xt_b, xr_b = _bits(xt), _bits(xr)
    n_chunk = CH * syn.HIDDEN
    for grp in (0, chunks, 2 * chunks - 1):
        S = ofp4.nvfp4_global_scale(ofp4.tensor_amax(xr_b[grp * n_chunk:(grp + 1) * n_chunk]))
        for r0, r1 in _samples(CH, span=16):
            _check_rows(NV, 1, xt_b, xr_b, syn.HIDDEN, grp * CH + r0, grp * CH + r1, S, g, y_g=y, y_r=g.y)
    del xt_b, xr_b
    sb, sf, n = G.oracle_plane_sums(xt, xr, y, g.y)
    a, b = acc.cpu().numpy(), acc_l.cpu().numpy()
    G.say(f"  one call {a.tolist()}, two calls {b.tolist()}, oracle {(sb, sf, n)}")
    assert a[2] == b[2] == n == xt.numel()
    assert G.rel_close(a[0], sb) and G.rel_close(a[1], sf), (a, (sb, sf))
    assert G.rel_close(b[0], sb) and G.rel_close(b[1], sf), (b, (sb, sf))


@pytest.mark.parametrize("bits", [2, 3])
def test_stream_layer_wider_records(bits):
    """The 2- and 3-bit records of one streamed layer as the benchmark times
    them: 17 chunks of [8192, 2048] in one single-pass encode (chunk scales,
    no rollout y), then guided_fake_quant with that record; sampled rows of
    three chunks against the oracle."""
    G.say(f"full size: streamed layer, bits {bits}, 17 x [8192, 2048]")
    layer, chunks, CH = 3, 17, syn.STREAM_CHUNK
    dev = G.DEV
    sigma = syn.stream_sigma(layer, dev)
    xt = torch.empty((chunks * CH, syn.HIDDEN), dtype=torch.bfloat16, device=dev)
    xr = torch.empty_like(xt)
    for c in range(chunks):
        a, b = syn.stream_pair(layer, c, dev, sigma=sigma)
        xt[c * CH:(c + 1) * CH].copy_(a)
        xr[c * CH:(c + 1) * CH].copy_(b)
    work = tq.quant_workspace(NV, chunks * CH, syn.HIDDEN, CH, device=dev)
    fails0 = tq.encode_wait_failures()
    g = tq.encode_guidance(xr, NV, bits, group_rows=CH, work=work)
    y, codes = tq.guided_fake_quant(xt, g, with_codes=True)
    torch.cuda.synchronize()
    assert tq.encode_wait_failures() == fails0
    xt_b, xr_b = _bits(xt), _bits(xr)
    n_chunk = CH * syn.HIDDEN
    for c in (0, 9, 16):
        S = ofp4.nvfp4_global_scale(ofp4.tensor_amax(xr_b[c * n_chunk:(c + 1) * n_chunk]))
        assert G.f32(g.gscale).reshape(chunks, 2)[c, 0] == S
        for r0, r1 in _samples(CH):
            _check_rows(NV, bits, xt_b, xr_b, syn.HIDDEN, c * CH + r0, c * CH + r1, S, g, y_g=y, codes_g=codes)


def test_whole_stream_encode_one_call():
    """The rollout side of the whole streamed workload in one call, as the
    benchmark's step runs it: 20 layers x 17 chunks of [8192, 2048] (340
    groups, one global scale each). Every group's {S, A} against the oracle's
    scale of the exact amax, every layer bit for bit against a call of its
    own, sampled rows of the first, middle and last group against the oracle."""
    G.say("full size: whole stream, 20 x 17 x [8192, 2048] in one encode call")
    layers, chunks, CH = len(syn.GUIDED_LAYERS), syn.STREAM_CHUNKS, syn.STREAM_CHUNK
    rows_l, cols = chunks * CH, syn.HIDDEN
    dev = G.DEV
    xr = torch.empty((layers, rows_l, cols), dtype=torch.bfloat16, device=dev)
    for li, layer in enumerate(syn.GUIDED_LAYERS):
        sigma = syn.stream_sigma(layer, dev)
        for c in range(chunks):
            _, b = syn.stream_pair(layer, c, dev, sigma=sigma)
            xr[li, c * CH:(c + 1) * CH].copy_(b)
            del b
    flat = xr.view(layers * rows_l, cols)
    work = tq.quant_workspace(NV, layers * rows_l, cols, CH, device=dev)
    fails0 = tq.encode_wait_failures()
    g = tq.encode_guidance(flat, NV, 1, group_rows=CH, work=work)
    torch.cuda.synchronize()
    G_ = layers * chunks
    assert tq.encode_wait_failures() == fails0
    # every group's amax (plain torch, exact) and the oracle's S of it
    amax = (flat.view(torch.int16) & 0x7FFF).view(G_, CH * cols).amax(dim=1).cpu().numpy().astype(np.uint16)
    A = ofp4.bf16_to_f32(amax)
    S = np.array([ofp4.nvfp4_global_scale(a) for a in A], np.float32)
    gs = G.f32(g.gscale).reshape(G_, 2)
    G.assert_same(gs[:, 1], A, "whole-stream A")
    G.assert_same(gs[:, 0], S, "whole-stream S")
    # each layer on its own gives the same planes and scales
    guide = g.guide.view(layers, rows_l, -1)
    scales = g.scales.view(layers, rows_l, -1)
    for li in range(layers):
        gl = tq.encode_guidance(xr[li], NV, 1, group_rows=CH)
        assert torch.equal(gl.guide, guide[li]), li
        assert torch.equal(gl.scales, scales[li]), li
        assert torch.equal(gl.gscale.view(-1), g.gscale.view(G_, 2)[li * chunks:(li + 1) * chunks].reshape(-1)), li
    B = ofp4.BLOCK[NV]
    for grp in (0, G_ // 2, G_ - 1):
        for r0, r1 in _samples(CH, span=32):
            a0, a1 = grp * CH + r0, grp * CH + r1
            xb = _bits(flat[a0:a1])
            o = ofp4.encode_guidance(NV, 1, xb, S[grp])
            G.assert_same(G.u8(g.guide[a0:a1]).reshape(-1), o["guide"], f"guide group {grp} rows {r0}:{r1}")
            G.assert_same(G.u8(g.scales[a0:a1]).reshape(-1), o["scales"], f"scales group {grp} rows {r0}:{r1}")
            assert o["scales"].size == (a1 - a0) * cols // B


def test_stream_layer_per_token_scales():
    """One streamed layer, 139,264 x 2048, with a global scale per token
    (group_rows = 1, the packed single-pass encode): every row's S against
    the oracle's amax of that row, sampled rows block by block, fused sums
    and mismatch counts against sums and counts over the library's outputs."""
    G.say("full size: streamed layer, per-token global scales")
    layer, chunks, CH = 20, 17, syn.STREAM_CHUNK
    dev = G.DEV
    sigma = syn.stream_sigma(layer, dev)
    xt = torch.empty((chunks * CH, syn.HIDDEN), dtype=torch.bfloat16, device=dev)
    xr = torch.empty_like(xt)
    for c in range(chunks):
        a, b = syn.stream_pair(layer, c, dev, sigma=sigma)
        xt[c * CH:(c + 1) * CH].copy_(a)
        xr[c * CH:(c + 1) * CH].copy_(b)
    rows, cols = xt.shape
    g = tq.encode_guidance(xr, NV, 1, with_y=True, group_rows=1)
    y, codes, acc, counts = tq.guided_fake_quant_stats(xt, xr, g, with_codes=True, mismatch=True)
    torch.cuda.synchronize()
    # every row's global scale
    amax_bits = (xr.view(torch.int16) & 0x7FFF).amax(dim=1).cpu().numpy().astype(np.uint16)
    A = ofp4.bf16_to_f32(amax_bits)
    S = np.array([ofp4.nvfp4_global_scale(a) for a in A], np.float32)
    gs = G.f32(g.gscale).reshape(rows, 2)
    G.assert_same(gs[:, 1], A, "per-token A")
    G.assert_same(gs[:, 0], S, "per-token S")
    xt_b, xr_b = _bits(xt), _bits(xr)
    for r0, r1 in _samples(rows, span=24):
        for r in range(r0, r1):
            _check_rows(NV, 1, xt_b, xr_b, cols, r, r + 1, S[r], g, y_g=y, codes_g=codes, y_r=g.y)
    sb, sf, n = G.oracle_plane_sums(xt, xr, y, g.y)
    a = acc.cpu().numpy()
    assert a[2] == n and G.rel_close(a[0], sb) and G.rel_close(a[1], sf), (a, (sb, sf, n))
    g4 = tq.encode_guidance(xr, NV, 4, group_rows=1)
    _, codes_rtn = tq.guided_fake_quant(xt, g, bits=0, with_codes=True)
    G.assert_same(counts.cpu().numpy(), G.oracle_plane_counts(codes, g4.guide, codes_rtn),
                  "mismatch counts, per-token scales")


@pytest.mark.parametrize("bits", [0, 1, 2, 3, 4])
def test_moe_layer_full_size(bits):
    """Routed-expert inputs of one MoE layer: 65,536 permuted rows x 2048,
    NVFP4, one global scale for the tensor."""
    G.say(f"full size: MoE layer [65536, 2048] bits={bits}")
    xt, xr, rows_token, _ = syn.moe_pair(20, device=G.DEV)
    rows, cols = xt.shape
    rec = 4 if bits == 0 else bits
    g = tq.encode_guidance(xr, NV, rec, with_y=True)
    y, codes = tq.guided_fake_quant(xt, g, bits=bits, with_codes=True)
    q = tq.quantize_rtn(xt, NV)
    torch.cuda.synchronize()
    xt_b, xr_b = _bits(xt), _bits(xr)
    S = _group_S(NV, xr_b)
    S_t = _group_S(NV, xt_b)
    assert G.f32(g.gscale)[0] == S
    assert G.f32(q.gscale)[0] == S_t
    for r0, r1 in _samples(rows):
        _check_rows(NV, rec, xt_b, xr_b, cols, r0, r1, S, g, y_g=y, codes_g=codes, y_r=g.y, gbits=bits)
        es = slice(r0 * cols, r1 * cols)
        oq = ofp4.quantize_rtn(NV, xt_b[es], S_t)
        G.assert_same(G.u8(q.codes).reshape(rows, -1)[r0:r1].reshape(-1), oq["codes"], "rtn codes")
        G.assert_same(_bits(q.y)[es], oq["y"], "rtn y")
    # duplicate routed rows (one token in 8 experts) give identical outputs
    order = torch.argsort(rows_token, stable=True)
    tok_sorted = rows_token[order]
    first = order[0::8]
    assert torch.equal(tok_sorted[0::8], tok_sorted[7::8])
    for k in range(1, 8):
        other = order[k::8]
        assert torch.equal(y[first].view(torch.int16), y[other].view(torch.int16))
        assert torch.equal(g.guide[first], g.guide[other])
        assert torch.equal(g.scales[first], g.scales[other])


@pytest.mark.parametrize("which", [0, 1])
def test_kv_full_size(which):
    """FP4 KV cache guidance: K or V of one layer as [65536, 256], NVFP4 block
    16 along head_dim, full codes (bits=4) and the 1-bit record."""
    G.say(f"full size: KV [65536, 256] which={which}")
    xt, xr = syn.kv_pair(20, which, device=G.DEV)
    rows, cols = xt.shape
    xt_b, xr_b = _bits(xt), _bits(xr)
    S = _group_S(NV, xr_b)
    for bits in (4, 1):
        g = tq.encode_guidance(xr, NV, bits, with_y=True)
        y, codes, acc = tq.guided_fake_quant_stats(xt, xr, g, with_codes=True)
        torch.cuda.synchronize()
        assert G.f32(g.gscale)[0] == S
        for r0, r1 in _samples(rows, span=256):
            _check_rows(NV, bits, xt_b, xr_b, cols, r0, r1, S, g, y_g=y, codes_g=codes, y_r=g.y)
        sb, sf, n = G.oracle_plane_sums(xt, xr, y, g.y)
        a = acc.cpu().numpy()
        assert a[2] == n and G.rel_close(a[0], sb) and G.rel_close(a[1], sf), (a, (sb, sf, n))


def test_kv_cache_one_call_over_all_layers():
    """The FP4 KV cache of 20 layers, K and V, as the benchmark times it: one
    encode (full codes, bits=4) over the 40 tensors of [65536, 256] with one
    global scale each, and one guided call. Every tensor's {S, A} against the
    oracle's scale of the exact amax; the encode and the guided outputs of
    every tensor bit for bit against calls of their own; sampled rows of the
    first and last tensor against the oracle."""
    G.say("full size: KV cache, 40 x [65536, 256] in one call")
    n_t, rows_t, cols = 40, 65536, 256
    kt = torch.empty((n_t, rows_t, cols), dtype=torch.bfloat16, device=G.DEV)
    kr = torch.empty_like(kt)
    for li in range(20):
        for which in (0, 1):
            a, b = syn.kv_pair(20 + li, which, device=G.DEV)
            kt[2 * li + which].copy_(a)
            kr[2 * li + which].copy_(b)
            del a, b
    ft, fr = kt.view(-1, cols), kr.view(-1, cols)
    work = tq.quant_workspace(NV, ft.shape[0], cols, rows_t, device=G.DEV)
    fails0 = tq.encode_wait_failures()
    g = tq.encode_guidance(fr, NV, 4, group_rows=rows_t, work=work)
    y, _ = tq.guided_fake_quant(ft, g, bits=4)
    torch.cuda.synchronize()
    assert tq.encode_wait_failures() == fails0
    amax = (fr.view(torch.int16) & 0x7FFF).view(n_t, -1).amax(dim=1).cpu().numpy().astype(np.uint16)
    A = ofp4.bf16_to_f32(amax)
    S = np.array([ofp4.nvfp4_global_scale(v) for v in A], np.float32)
    gs = G.f32(g.gscale).reshape(n_t, 2)
    G.assert_same(gs[:, 1], A, "KV A")
    G.assert_same(gs[:, 0], S, "KV S")
    guide = g.guide.view(n_t, rows_t, -1)
    scales = g.scales.view(n_t, rows_t, -1)
    yv = y.view(n_t, rows_t, cols)
    for i in range(n_t):
        gi = tq.encode_guidance(kr[i], NV, 4)
        yi, _ = tq.guided_fake_quant(kt[i], gi, bits=4)
        assert torch.equal(gi.guide, guide[i]), i
        assert torch.equal(gi.scales, scales[i]), i
        assert torch.equal(gi.gscale.view(-1), g.gscale.view(n_t, 2)[i]), i
        assert torch.equal(yi.view(torch.int16), yv[i].view(torch.int16)), i
    for i in (0, n_t - 1):
        xt_b, xr_b = _bits(kt[i]), _bits(kr[i])
        gi = tq.encode_guidance(kr[i], NV, 4)
        for r0, r1 in _samples(rows_t, span=256):
            _check_rows(NV, 4, xt_b, xr_b, cols, r0, r1, S[i], gi, y_g=yv[i])


def test_mxfp4_full_size_with_ties():
    """MXFP4 W4A4: [65536, 2048] pairs with 0.1% of the elements exactly on
    E2M1 rounding midpoints; every record width (1 to 4 bits) with guided
    rounding, Reconstruct alone for 1 to 3 bits and RTN under the rollout
    scales, on sampled rows against the oracle."""
    G.say("full size: MXFP4 [65536, 2048] with midpoint ties")
    xt, xr = syn.mxfp4_pair(device=G.DEV)
    rows, cols = xt.shape
    xt_b, xr_b = _bits(xt), _bits(xr)
    q = tq.quantize_rtn(xt, MX)
    torch.cuda.synchronize()
    for bits in (1, 2, 3, 4):
        g = tq.encode_guidance(xr, MX, bits, with_y=True)
        y, codes = tq.guided_fake_quant(xt, g, with_codes=True)
        ref = tq.decode_guidance(xt, g) if bits < 4 else None
        y0, codes0 = tq.guided_fake_quant(xt, g, bits=0, with_codes=True) if bits == 1 else (None, None)
        torch.cuda.synchronize()
        for r0, r1 in _samples(rows):
            o = _check_rows(MX, bits, xt_b, xr_b, cols, r0, r1, None, g, y_g=y, codes_g=codes, y_r=g.y)
            es = slice(r0 * cols, r1 * cols)
            if ref is not None:
                od = ofp4.decode_guidance(MX, xt_b[es], o["guide"], o["scales"], None, bits=bits)
                G.assert_same(G.u8(ref).reshape(-1)[r0 * cols // 2:r1 * cols // 2], od,
                              f"mx decode bits {bits} rows {r0}:{r1}")
            if y0 is not None:
                _check_rows(MX, bits, xt_b, xr_b, cols, r0, r1, None, g, y_g=y0, codes_g=codes0, gbits=0)
    for r0, r1 in _samples(rows):
        es = slice(r0 * cols, r1 * cols)
        oq = ofp4.quantize_rtn(MX, xt_b[es])
        G.assert_same(G.u8(q.codes).reshape(rows, -1)[r0:r1].reshape(-1), oq["codes"], "mx rtn codes")
        G.assert_same(_bits(q.y)[es], oq["y"], "mx rtn y")
    # the sampled rows hold injected ties (t exactly on an E2M1 midpoint)
    n_ties = 0
    for r0, r1 in _samples(rows):
        es = slice(r0 * cols, r1 * cols)
        sc = ofp4.mxfp4_block_scales(xt_b[es])
        _, r = ofp4.mxfp4_block_factors(sc)
        t = ofp4.normalize(xt_b[es], r, 32)
        n_ties += int(np.isin(t, np.array(syn.MIDPOINT_MULTIPLES, np.float32)).sum())
    assert n_ties > 100, n_ties


def test_tiny_pair_whole_tensor():
    """The tiny NVFP4 pair (256 x 2048, seed 0): every call, whole tensor."""
    G.say("tiny pair, whole tensor")
    xt, xr = syn.tiny_pair()
    xt_b, xr_b = syn.bits_u16(xt).reshape(-1), syn.bits_u16(xr).reshape(-1)
    G.check_quantize(xt_b, 256, 2048, NV)
    for bits in (1, 4):
        G.check_encode(xr_b, 256, 2048, NV, bits)
        G.check_guided_stats(xt_b, xr_b, 256, 2048, NV, bits)
    G.check_guided(xt_b, xr_b, 256, 2048, NV, 0)
    G.check_decode(xt_b, xr_b, 256, 2048, NV)


def test_moe_layer_per_expert_scales():
    """The MoE layer [65536, 2048] with one global scale per expert (256
    experts, offsets straight from routing): every expert's S against the
    oracle's amax of its rows; experts sampled whole against the oracle."""
    G.say("full size: MoE layer, per-expert scales")
    xt, xr, _, offsets = syn.moe_pair(20, device=G.DEV)
    rows, cols = xt.shape
    g = tq.encode_guidance_grouped(xr, offsets, NV, 1, with_y=True)
    y, codes = tq.guided_fake_quant(xt, g, with_codes=True)
    torch.cuda.synchronize()
    offs = offsets.cpu().numpy()
    amax = (xr.view(torch.int16) & 0x7FFF).amax(dim=1).cpu().numpy().astype(np.uint16)
    gs = G.f32(g.gscale).reshape(-1, 2)
    xt_b, xr_b = _bits(xt), _bits(xr)
    for e in range(len(offs) - 1):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        A = ofp4.bf16_to_f32(amax[r0:r1]).max() if r1 > r0 else np.float32(0)
        assert gs[e, 1] == A and gs[e, 0] == ofp4.nvfp4_global_scale(A), e
    for e in (0, 1, 77, 128, 255):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        es = slice(r0 * cols, r1 * cols)
        o = ofp4.encode_guidance(NV, 1, xr_b[es])
        og = ofp4.guided_fake_quant(NV, 1, xt_b[es], o["guide"], o["scales"], o["gscale"])
        G.assert_same(G.u8(g.guide).reshape(-1)[r0 * cols // 8:r1 * cols // 8], o["guide"], f"expert {e} guide")
        G.assert_same(G.u8(g.scales).reshape(-1)[r0 * cols // 16:r1 * cols // 16], o["scales"], "scales")
        G.assert_same(_bits(g.y)[es], o["y"], f"expert {e} rollout y")
        G.assert_same(_bits(y)[es], og["y"], f"expert {e} guided y")
        G.assert_same(G.u8(codes).reshape(-1)[r0 * cols // 2:r1 * cols // 2], og["codes"], "guided codes")
