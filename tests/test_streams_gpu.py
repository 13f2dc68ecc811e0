"""Streams and graphs: calls on two streams at once give the results of the
same calls run one after another, and the step captured in a HIP graph gives,
on every replay, the eager results (the library clears its flags with a
kernel, not a memset, so captures replay correctly)."""

import pytest
import torch

import precision_rl_nvfp4_amd as tq
import synthetic as syn
from tests import _gpu as G

pytestmark = pytest.mark.gpu

CH = syn.STREAM_CHUNK


def _chunks(layer, n):
    a = [syn.stream_pair(layer, c, G.DEV) for c in range(n)]
    return torch.cat([p[0] for p in a]), torch.cat([p[1] for p in a])


def test_single_pass_encodes_on_two_streams():
    """Two encodes of 2 x [8192, 2048] chunks (each needs every CU resident
    for its single pass), enqueued on two streams before any sync: both
    finish with the sequential results and no wait gives up."""
    G.say("two streams: single-pass encodes")
    xa = _chunks(20, 2)[1]
    xb = _chunks(21, 2)[1]
    rows, cols = xa.shape
    wa = tq.quant_workspace("nvfp4", rows, cols, CH, device=G.DEV)
    wb = tq.quant_workspace("nvfp4", rows, cols, CH, device=G.DEV)
    ref_a = tq.encode_guidance(xa, "nvfp4", 1, with_y=True, group_rows=CH)
    ref_b = tq.encode_guidance(xb, "nvfp4", 1, with_y=True, group_rows=CH)
    torch.cuda.synchronize()
    fails0 = tq.encode_wait_failures()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(sa):
            ga = tq.encode_guidance(xa, "nvfp4", 1, with_y=True, group_rows=CH, work=wa)
        with torch.cuda.stream(sb):
            gb = tq.encode_guidance(xb, "nvfp4", 1, with_y=True, group_rows=CH, work=wb)
        outs.append((ga, gb))
    torch.cuda.synchronize()
    for ga, gb in outs:
        for g, ref in ((ga, ref_a), (gb, ref_b)):
            assert torch.equal(g.guide, ref.guide) and torch.equal(g.scales, ref.scales)
            assert torch.equal(g.gscale, ref.gscale)
            assert torch.equal(g.y.view(torch.int16), ref.y.view(torch.int16))
    # the launches were ordered on the device: none waited on the other
    assert tq.encode_wait_failures() == fails0


@pytest.mark.parametrize("n_chunks", [1, 4])
def test_guided_calls_on_two_streams(n_chunks):
    """Guided calls on two streams at once, each with its own workspace: a
    fused pass and a plain one, then two fused passes (4 chunks: 8,192
    tiles, so each call's final sum is split over eight workgroups with its
    own ticket counter). Every result equals the sequential one."""
    G.say(f"two streams: guided calls, {n_chunks} chunks")
    xt, xr = _chunks(22, n_chunks)
    g = tq.encode_guidance(xr, "nvfp4", 1, group_rows=CH)
    ref_y, ref_c, ref_acc = tq.guided_fake_quant_stats(xt, xr, g, with_codes=True)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(sa):
        ya, ca, acc_a = tq.guided_fake_quant_stats(xt, xr, g, with_codes=True)
    with torch.cuda.stream(sb):
        yb, cb = tq.guided_fake_quant(xt, g, with_codes=True)
        yc, cc, acc_c = tq.guided_fake_quant_stats(xt, xr, g, with_codes=True)
    torch.cuda.synchronize()
    assert torch.equal(ya.view(torch.int16), ref_y.view(torch.int16)) and torch.equal(ca, ref_c)
    assert torch.equal(yb.view(torch.int16), ref_y.view(torch.int16)) and torch.equal(cb, ref_c)
    assert torch.equal(yc.view(torch.int16), ref_y.view(torch.int16)) and torch.equal(cc, ref_c)
    assert torch.equal(acc_a, ref_acc) and torch.equal(acc_c, ref_acc)


@pytest.mark.parametrize("n_chunks", [2, 5])
def test_step_captured_in_a_graph(n_chunks):
    """encode (single pass) + guided_fake_quant_stats with mismatch counts on
    2 chunks (4,096 tiles: the final sum in one workgroup) and 5 (10,240
    tiles: split over eight, whose ticket counter the guided kernel zeroes on
    every replay), captured once, replayed 4 times with eager work in
    between; every replay equals the eager results."""
    G.say(f"graph capture of the step, {n_chunks} chunks")
    xt, xr = _chunks(23, n_chunks)
    rows, cols = xt.shape
    eager_g = tq.encode_guidance(xr, "nvfp4", 1, group_rows=CH)
    eager = tq.guided_fake_quant_stats(xt, xr, eager_g, with_codes=True, mismatch=True)
    torch.cuda.synchronize()
    fails0 = tq.encode_wait_failures()
    # static buffers
    work = tq.quant_workspace("nvfp4", rows, cols, CH, device=G.DEV)
    swork = tq.guided_stats_workspace("nvfp4", rows, cols, CH, device=G.DEV)
    guide = torch.empty_like(eager_g.guide)
    scales = torch.empty_like(eager_g.scales)
    gsc = torch.empty_like(eager_g.gscale)
    y = torch.empty_like(xt)
    codes = torch.empty_like(eager[1])
    acc = torch.empty(3, dtype=torch.float64, device=G.DEV)
    cnt = torch.empty(32, dtype=torch.int64, device=G.DEV)

    def step():
        g = tq.encode_guidance(xr, "nvfp4", 1, group_rows=CH, guide=guide, scales=scales, gscale_out=gsc,
                               work=work)
        tq.guided_fake_quant_stats(xt, xr, g, with_codes=True, acc=acc, y=y, codes=codes, work=swork,
                                   counts=cnt)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in (guide, scales, y, codes):
            t.zero_()
        acc.fill_(-1.0)
        cnt.fill_(-1)
        gsc.fill_(0.0)
        graph.replay()
        torch.cuda.synchronize()
        # eager work between replays
        _ = tq.encode_guidance(xt, "nvfp4", 4, group_rows=CH)
        torch.cuda.synchronize()
        assert torch.equal(guide, eager_g.guide) and torch.equal(scales, eager_g.scales), rep
        assert torch.equal(gsc, eager_g.gscale), rep
        assert torch.equal(y.view(torch.int16), eager[0].view(torch.int16)), rep
        assert torch.equal(codes, eager[1]), rep
        assert torch.equal(acc, eager[2]), rep
        assert torch.equal(cnt, eager[3]), rep
        assert tq.encode_wait_failures() == fails0, rep
