"""The single-pass encode's bounded waits, forced from the host: with a wait
limit of one poll the workgroups give up at once instead of waiting for each
other's tile maxima and scales. The launch must still complete and count
its failures in the workspace; with the limit restored the next call on the
same workspace is exact again (bit-identical to a call made before)."""

import pytest
import torch

import precision_rl_nvfp4_amd as tq
import synthetic as syn
from precision_rl_nvfp4_amd import _abi
from tests import _gpu as G

pytestmark = pytest.mark.gpu

NV = tq.NVFP4


def test_waits_give_up_and_the_next_call_recovers():
    G.say("single-pass encode with a wait limit of 1 poll, then the default")
    lib = _abi.load()
    CH, chunks, cols = syn.STREAM_CHUNK, 2, syn.HIDDEN
    sigma = syn.stream_sigma(20, G.DEV)
    xr = torch.cat([syn.stream_pair(20, c, G.DEV, sigma=sigma)[1] for c in range(chunks)])
    rows = xr.shape[0]
    work = tq.quant_workspace(NV, rows, cols, CH, device=G.DEV)
    fails = work.view(torch.int32)[chunks * 2048]
    ref = tq.encode_guidance(xr, NV, 1, group_rows=CH, work=work)
    torch.cuda.synchronize()
    assert fails.item() == 0
    prev = lib.trace_set_wait_limit(1)
    try:
        tq.encode_guidance(xr, NV, 1, group_rows=CH, work=work)
        torch.cuda.synchronize()
        assert fails.item() > 0
    finally:
        assert lib.trace_set_wait_limit(prev) == 1
    g = tq.encode_guidance(xr, NV, 1, group_rows=CH, work=work)
    torch.cuda.synchronize()
    assert fails.item() == 0
    assert torch.equal(g.guide, ref.guide)
    assert torch.equal(g.scales, ref.scales)
    assert torch.equal(g.gscale, ref.gscale)
