"""Straight-through autograd ops on the GPU (Algorithm 1 prose: the forward
value is the guided FP4 value, the gradient reaches the unquantized input
unchanged): forward values bit-exact against the oracle, backward the
identity, and a small QAT forward/backward through the guided-layer policy."""

import pytest
import torch

import precision_rl_nvfp4_amd as tq
import synthetic as syn
from oracle import fp4 as ofp4
from precision_rl_nvfp4_amd import ste
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _pair(rows, cols, seed):
    xt, xr = syn.activation_pair(rows, cols, (92, seed))
    return xt, xr


@pytest.mark.parametrize("bits", [1, 4])
def test_guided_ste_forward_and_identity_backward(bits):
    G.say(f"STE guided bits={bits}")
    xt, xr = _pair(74, 2048, bits)
    t = xt.to(G.DEV).reshape(2, 37, 2048).requires_grad_(True)
    r = xr.to(G.DEV)
    g = tq.encode_guidance(r, "nvfp4", bits)
    y = ste.guided_fake_quant_ste(t, g)
    assert y.shape == t.shape and y.dtype == torch.bfloat16
    bt, br = syn.bits_u16(xt).reshape(-1), syn.bits_u16(xr).reshape(-1)
    o_enc = ofp4.encode_guidance(ofp4.NVFP4, bits, br)
    o = ofp4.guided_fake_quant(ofp4.NVFP4, bits, bt, o_enc["guide"], o_enc["scales"], o_enc["gscale"])
    G.assert_same(G.bits_of(y), o["y"], "STE forward")
    up = torch.randn(t.shape, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).to(G.DEV)
    y.backward(up)
    assert torch.equal(t.grad.view(torch.int16), up.view(torch.int16))


def test_rtn_ste_forward_and_identity_backward():
    G.say("STE rtn")
    xt, _ = _pair(64, 256, 3)
    t = xt.to(G.DEV).requires_grad_(True)
    y = ste.rtn_fake_quant_ste(t, "nvfp4")
    o = ofp4.quantize_rtn(ofp4.NVFP4, syn.bits_u16(xt).reshape(-1))
    G.assert_same(G.bits_of(y), o["y"], "RTN STE forward")
    y.float().sum().backward()
    assert torch.equal(t.grad, torch.ones_like(t))


def test_qat_step_through_policy():
    """Two layers, one guided and one not: the forward uses the guided value
    on the guided layer and RTN elsewhere; the input gradients equal those of
    the same network with the quantizers replaced by identities evaluated at
    the quantized values (float32 reference on the CPU)."""
    G.say("STE QAT step")
    rows, cols = 64, 256
    xt, xr = _pair(rows, cols, 5)
    W = torch.randn(cols, 32, generator=torch.Generator().manual_seed(2)) * 0.05
    qat = ste.GuidedQAT(num_layers=2, keep=1)
    r = xr.to(G.DEV)
    qat.put("act", 1, tq.encode_guidance(r, "nvfp4", 1))
    grads, outs = [], []
    for layer in (0, 1):
        t = xt.to(G.DEV).requires_grad_(True)
        q = qat(t, layer, "act")
        out = q.float() @ W.to(G.DEV)
        loss = (out * out).sum()
        loss.backward()
        grads.append(t.grad.float().cpu())
        outs.append(q.detach())
    bt = syn.bits_u16(xt).reshape(-1)
    o_rtn = ofp4.quantize_rtn(ofp4.NVFP4, bt)
    o_enc = ofp4.encode_guidance(ofp4.NVFP4, 1, syn.bits_u16(xr).reshape(-1))
    o_g = ofp4.guided_fake_quant(ofp4.NVFP4, 1, bt, o_enc["guide"], o_enc["scales"], o_enc["gscale"])
    G.assert_same(G.bits_of(outs[0]), o_rtn["y"], "layer 0 (RTN)")
    G.assert_same(G.bits_of(outs[1]), o_g["y"], "layer 1 (guided)")
    for layer in (0, 1):
        q = outs[layer].float().cpu()
        ref = ((2.0 * (q @ W)) @ W.t()).to(torch.bfloat16).float()
        assert torch.allclose(grads[layer], ref, rtol=2e-2, atol=1e-6), layer
