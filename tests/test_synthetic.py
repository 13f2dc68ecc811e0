"""The seeded input generators: shapes, determinism and the distribution
features the workloads call for (heavy tails, channel scales, routing, KV
outlier channels, exact midpoints)."""

import numpy as np
import torch

import synthetic as syn
from oracle import fp4


def test_tiny_pair_deterministic_and_shaped():
    a_t, a_r = syn.tiny_pair()
    b_t, b_r = syn.tiny_pair()
    assert a_t.shape == (256, 2048) and a_t.dtype == torch.bfloat16
    assert torch.equal(a_t.view(torch.int16), b_t.view(torch.int16))
    assert torch.equal(a_r.view(torch.int16), b_r.view(torch.int16))
    rel = ((a_r.float() - a_t.float()) / a_t.float()).nan_to_num(0)
    assert 0.005 < rel.std().item() < 0.02          # rollout = train * (1 + N(0, 0.01))


def test_student_t4_tails():
    g = syn._gen("cpu", 99)
    x = syn._student_t4((1_000_000,), g, "cpu")
    assert abs(x.var().item() - 2.0) < 0.2           # nu / (nu - 2)
    assert (x.abs() > 8).float().mean().item() > 1e-3   # heavy tail (normal: ~1e-15)


def test_moe_routing_structure():
    rows_token, offsets = syn.moe_routing(512, 20)
    assert rows_token.numel() == 512 * 8 and offsets[-1].item() == 512 * 8
    # every token appears exactly top-8 times, rows grouped by expert
    assert torch.equal(torch.bincount(rows_token, minlength=512), torch.full((512,), 8))
    xt, xr, rt, off = syn.moe_pair(20, tokens=256)
    assert xt.shape == (2048, 2048)
    # duplicated tokens give identical rows
    first = {}
    for i, t in enumerate(rt.tolist()):
        if t in first:
            assert torch.equal(xt[i].view(torch.int16), xt[first[t]].view(torch.int16))
            break
        first[t] = i


def test_kv_outlier_channels():
    xt, xr = syn.kv_pair(20, 0, tokens=1024)
    assert xt.shape == (2048, 256)
    per_chan = xt.float().reshape(1024, 512).abs().mean(0)
    big = (per_chan > 5).sum().item()
    assert big == 5


def test_mxfp4_midpoints_injected():
    xt, xr = syn.mxfp4_pair(rows=64, cols=2048, frac=0.01)
    for x in (xt, xr):
        b = syn.bits_u16(x)
        q = fp4.quantize_rtn(fp4.MXFP4, b)
        d, r = fp4.mxfp4_block_factors(q["scales"])
        t = fp4.normalize(b, r, 32)
        mids = np.isin(t, np.array(syn.MIDPOINT_MULTIPLES, dtype=np.float32))
        assert mids.mean() > 0.008


def test_stream_chunks_share_layer_scales():
    s1 = syn.stream_sigma(25)
    s2 = syn.stream_sigma(25)
    assert torch.equal(s1, s2)
    a, _ = syn.stream_pair(25, 0, rows=64, sigma=s1)
    b, _ = syn.stream_pair(25, 1, rows=64, sigma=s1)
    assert not torch.equal(a.view(torch.int16), b.view(torch.int16))
