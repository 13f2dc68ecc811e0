"""The single-pass encode's bounded waits, forced from the host: with a wait
limit of one poll nearly every wait gives up at once instead of waiting for
other workgroups' tile maxima and scales. A wait that gives up takes what it
waited for from the input itself, so every output must still be bit-identical
to the same call with the default limit, and the device's give-up count must
have grown. Two launch shapes: one group in flight at a time (8192-row
chunks) and several (1024-row groups)."""

import numpy as np
import pytest
import torch

import precision_rl_nvfp4_amd as tq
import synthetic as syn
from oracle import fp4 as ofp4
from precision_rl_nvfp4_amd import _abi
from tests import _gpu as G

pytestmark = pytest.mark.gpu

NV = tq.NVFP4


def _stream_rows(layer, chunks):
    sigma = syn.stream_sigma(layer, G.DEV)
    return torch.cat([syn.stream_pair(layer, c, G.DEV, sigma=sigma)[1] for c in range(chunks)])


@pytest.mark.parametrize("group_rows,chunks,bits", [(8192, 2, 1), (1024, 2, 4)])
def test_waits_give_up_and_results_stay_exact(group_rows, chunks, bits):
    G.say(f"single-pass encode, wait limit 1 poll: group_rows={group_rows} chunks={chunks} bits={bits}")
    lib = _abi.load()
    xr = _stream_rows(20, chunks)
    rows, cols = xr.shape
    work = tq.quant_workspace(NV, rows, cols, group_rows, device=G.DEV)
    ref = tq.encode_guidance(xr, NV, bits, with_y=True, group_rows=group_rows, work=work)
    torch.cuda.synchronize()
    fails0 = tq.encode_wait_failures()
    prev = lib.trace_set_wait_limit(1)
    try:
        g = tq.encode_guidance(xr, NV, bits, with_y=True, group_rows=group_rows, work=work)
        torch.cuda.synchronize()
    finally:
        assert lib.trace_set_wait_limit(prev) == 1
    fails1 = tq.encode_wait_failures()
    G.say(f"  waits that gave up: {fails1 - fails0}")
    assert fails1 > fails0
    assert torch.equal(g.guide, ref.guide)
    assert torch.equal(g.scales, ref.scales)
    assert torch.equal(g.gscale, ref.gscale)
    assert torch.equal(g.y.view(torch.int16), ref.y.view(torch.int16))
    # and against the oracle's scales of the exact amax of every group
    gs = G.f32(g.gscale).reshape(-1, 2)
    amax = (xr.view(torch.int16) & 0x7FFF).view(rows // group_rows, -1).amax(dim=1).cpu().numpy()
    A = ofp4.bf16_to_f32(amax.astype(np.uint16))
    G.assert_same(gs[:, 1], A, "A after give-ups")
    G.assert_same(gs[:, 0], np.array([ofp4.nvfp4_global_scale(a) for a in A], np.float32), "S after give-ups")
    # the default limit again: no give-up, same results
    g2 = tq.encode_guidance(xr, NV, bits, with_y=True, group_rows=group_rows, work=work)
    torch.cuda.synchronize()
    assert tq.encode_wait_failures() == fails1
    assert torch.equal(g2.guide, ref.guide) and torch.equal(g2.gscale, ref.gscale)


def test_row_offset_single_pass_gives_up_exactly():
    """The single pass over row-offset groups (one S per expert of a routed
    MoE layer) at a wait limit of one poll: bit-identical to the default."""
    G.say("row-offset single pass, wait limit 1 poll")
    lib = _abi.load()
    _, xr, _, offsets = syn.moe_pair(21, tokens=2048, device=G.DEV)
    ref = tq.encode_guidance_grouped(xr, offsets, NV, 1, with_y=True)
    torch.cuda.synchronize()
    fails0 = tq.encode_wait_failures()
    prev = lib.trace_set_wait_limit(1)
    try:
        g = tq.encode_guidance_grouped(xr, offsets, NV, 1, with_y=True)
        torch.cuda.synchronize()
    finally:
        assert lib.trace_set_wait_limit(prev) == 1
    G.say(f"  waits that gave up: {tq.encode_wait_failures() - fails0}")
    assert tq.encode_wait_failures() > fails0
    assert torch.equal(g.guide, ref.guide) and torch.equal(g.scales, ref.scales)
    assert torch.equal(g.gscale, ref.gscale)
    assert torch.equal(g.y.view(torch.int16), ref.y.view(torch.int16))
