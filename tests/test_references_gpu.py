"""The measurement references of the library (trace_stream_copy,
trace_stream_mix): they must move exactly the bytes they claim to, or the
rates the benchmark reports beside the kernels would be measured on the
wrong traffic. Checked against torch's copy and XOR on random bytes, at a
size that spans many workgroup tiles and ends in a partial tile."""

import pytest
import torch

import precision_rl_nvfp4_amd as tq
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _bytes(n, seed):
    g = torch.Generator(device=G.DEV)
    g.manual_seed(seed)
    return torch.randint(0, 256, (n,), dtype=torch.uint8, device=G.DEV, generator=g)


@pytest.mark.parametrize("n", [16, 16 * (2048 * 37 + 5), 1 << 24])
def test_stream_copy_and_mix(n):
    G.say(f"stream references: {n} bytes")
    a, b = _bytes(n, 1), _bytes(n, 2)
    out = torch.full((n + 64,), 0xA5, dtype=torch.uint8, device=G.DEV)   # canary past the end
    tq.stream_copy(a, out[:n])
    torch.cuda.synchronize()
    assert torch.equal(out[:n], a)
    assert bool((out[n:] == 0xA5).all())
    tq.stream_mix(a, b, out[:n])
    torch.cuda.synchronize()
    assert torch.equal(out[:n], a ^ b)
    assert bool((out[n:] == 0xA5).all())


def test_stream_references_empty():
    e = torch.empty(0, dtype=torch.uint8, device=G.DEV)
    tq.stream_copy(e, e.clone())
    tq.stream_mix(e, e.clone(), e.clone())
    torch.cuda.synchronize()
