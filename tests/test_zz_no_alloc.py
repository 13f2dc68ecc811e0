"""encode_guidance_noalloc, the entry point that allocates nothing (its
workspace is the library's own per-device scratch array), against
encode_guidance with a caller workspace, through the C ABI, bit for bit.

The calls run in a row on the same device, so each one finds the scratch
array as the previous one left it: a larger single-pass encode first, then a
smaller one with more groups in flight, then the two-pass schedule, then
calls that need no workspace at all."""

import ctypes

import pytest
import torch

import precision_rl_nvfp4_amd as tq
import synthetic as syn
from precision_rl_nvfp4_amd import _abi
from tests import _gpu as G

pytestmark = pytest.mark.gpu

NV, MX = tq.NVFP4, tq.MXFP4


def _p(t):
    return None if t is None else t.data_ptr()


def _noalloc(x, fmt, bits, group_rows, with_y):
    """encode_guidance_noalloc through the raw C ABI into fresh buffers."""
    rows, cols = x.shape
    G_ = rows // group_rows if group_rows else 1
    guide = torch.full((rows, cols * bits // 8), 0xA5, dtype=torch.uint8, device=G.DEV)
    scales = torch.full((rows, cols // tq.BLOCK[fmt]), 0xA5, dtype=torch.uint8, device=G.DEV)
    gs = torch.full((G_, 2), -7.0, dtype=torch.float32, device=G.DEV) if fmt == NV else None
    y = torch.full((rows, cols), -1.0, dtype=torch.bfloat16, device=G.DEV) if with_y else None
    st = _abi.load().encode_guidance_noalloc(fmt, bits, rows, cols, group_rows, _p(x), None, _p(guide),
                                             _p(scales), _p(gs), _p(y),
                                             torch.cuda.current_stream().cuda_stream)
    assert st == _abi.OK, _abi.status_str(st)
    return guide, scales, gs, y


def _rows(layer, nrows):
    sigma = syn.stream_sigma(layer, G.DEV)
    parts, have, c = [], 0, 0
    while have < nrows:
        _, xr = syn.stream_pair(layer, c, G.DEV, sigma=sigma)
        parts.append(xr[: nrows - have])
        have += parts[-1].shape[0]
        c += 1
    return torch.cat(parts).contiguous()


CASES = [  # (fmt, bits, rows, group_rows, with_y): in call order, the second smaller than the first
    (NV, 1, 4 * 8192, 8192, True),     # single pass, one group in flight
    (NV, 4, 6 * 1024, 1024, True),     # single pass, six groups in flight (smaller input)
    (NV, 2, 2048, 0, False),           # one group: two passes
    (NV, 3, 512, 1, True),             # one S per token: packed, no workspace
    (MX, 1, 256, 0, True),             # MXFP4: no global scale, no workspace
]


def test_noalloc_equals_workspace_call_in_a_row():
    fails0 = tq.encode_wait_failures()
    for i, (fmt, bits, rows, gr, with_y) in enumerate(CASES):
        G.say(f"noalloc call {i}: fmt={fmt} bits={bits} rows={rows} group_rows={gr}")
        x = _rows(20 + i, rows)
        got = _noalloc(x, fmt, bits, gr, with_y)
        ref = tq.encode_guidance(x, fmt, bits, with_y=with_y, group_rows=gr)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref.guide), i
        assert torch.equal(got[1], ref.scales), i
        if fmt == NV:
            assert torch.equal(got[2], ref.gscale), i
        if with_y:
            assert torch.equal(got[3].view(torch.int16), ref.y.view(torch.int16)), i
    assert tq.encode_wait_failures() == fails0


def test_noalloc_repeated_on_one_input_and_captured():
    """The same call twice more on the first case's input (the scratch now
    holds the last call's words), then captured in a graph and replayed with
    eager calls between replays: every result equals the workspace call."""
    G.say("noalloc: repeated calls and a graph capture")
    x = _rows(30, 2 * 8192)
    rows, cols = x.shape
    ref = tq.encode_guidance(x, NV, 1, with_y=True, group_rows=8192)
    for _ in range(2):
        got = _noalloc(x, NV, 1, 8192, True)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref.guide) and torch.equal(got[1], ref.scales)
        assert torch.equal(got[2], ref.gscale) and torch.equal(got[3].view(torch.int16), ref.y.view(torch.int16))
    guide = torch.empty_like(ref.guide)
    scales = torch.empty_like(ref.scales)
    gs = torch.empty_like(ref.gscale)
    y = torch.empty_like(ref.y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        tq.encode_guidance_noalloc(x, "nvfp4", 1, group_rows=8192, guide=guide, scales=scales, gscale_out=gs, y=y)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tq.encode_guidance_noalloc(x, "nvfp4", 1, group_rows=8192, guide=guide, scales=scales, gscale_out=gs, y=y)
    small = _rows(31, 1024)
    for rep in range(3):
        for t in (guide, scales, y):
            t.zero_()
        gs.fill_(0.0)
        graph.replay()
        torch.cuda.synchronize()
        _noalloc(small, NV, 4, 256, False)      # eager use of the scratch between replays
        torch.cuda.synchronize()
        assert torch.equal(guide, ref.guide) and torch.equal(scales, ref.scales), rep
        assert torch.equal(gs, ref.gscale), rep
        assert torch.equal(y.view(torch.int16), ref.y.view(torch.int16)), rep
