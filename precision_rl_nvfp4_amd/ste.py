"""Training-side use of the guided path: straight-through autograd ops and the
guided-layer policy.

Paper: "TRACE: Rollout-Guided Quantization-Aware Training for FP4
Reinforcement Learning of MoE Language Models".
  * Algorithm 1 prose: the forward value is the guided FP4 value, and STE
    returns its second argument in the forward pass while the gradient goes
    to its first argument (the unquantized activation) unchanged.
  * §3.2 "Key Design" and §4.3 "Modular Sensitivity Study": the record is
    kept for the deepest layers only (the latter half by default; 40, 20, 10
    or 5 of 40 layers are compared); the other layers use vanilla FP4 fake
    quantization with their own scales.

Both ops call the C ABI through the binding; the backward pass is the
identity, so it launches nothing.
"""

from __future__ import annotations

from typing import Dict, Hashable, Optional, Sequence

import torch

from . import Guidance, guided_fake_quant, quantize_rtn

__all__ = ["GuidedFakeQuantSTE", "RTNFakeQuantSTE", "guided_fake_quant_ste", "rtn_fake_quant_ste",
           "guided_layers", "GuidedQAT"]


def _as_rows(x: torch.Tensor) -> torch.Tensor:
    """[..., cols] -> [rows, cols] view (the calls quantize along the last dim)."""
    if x.dim() < 1:
        raise ValueError("fake quantization needs at least one dimension")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    return x.reshape(-1, x.shape[-1])


class GuidedFakeQuantSTE(torch.autograd.Function):
    """y = guided FP4 value of x under the rollout record (forward);
    dL/dx = dL/dy (backward)."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, g: Guidance, bits: Optional[int]):
        y, _ = guided_fake_quant(_as_rows(x.detach()), g, bits=bits)
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, grad_y: torch.Tensor):
        return grad_y, None, None


class RTNFakeQuantSTE(torch.autograd.Function):
    """y = vanilla FP4 fake quantization of x with its own scales (forward);
    dL/dx = dL/dy (backward)."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, fmt, group_rows: int):
        q = quantize_rtn(_as_rows(x.detach()), fmt, group_rows=group_rows)
        return q.y.view(x.shape)

    @staticmethod
    def backward(ctx, grad_y: torch.Tensor):
        return grad_y, None, None


def guided_fake_quant_ste(x: torch.Tensor, g: Guidance, bits: Optional[int] = None) -> torch.Tensor:
    """Rollout-guided fake quantization with a straight-through gradient.
    x: contiguous bf16 [..., cols] whose rows match the record's."""
    return GuidedFakeQuantSTE.apply(x, g, bits)


def rtn_fake_quant_ste(x: torch.Tensor, fmt="nvfp4", group_rows: int = 0) -> torch.Tensor:
    """Vanilla FP4 fake quantization (own scales) with a straight-through gradient."""
    return RTNFakeQuantSTE.apply(x, fmt, group_rows)


def guided_layers(num_layers: int, keep: Optional[int] = None) -> range:
    """Indices of the layers whose rollout records are kept: the deepest
    `keep` of `num_layers` (default: the latter half)."""
    if num_layers < 0:
        raise ValueError("num_layers must be >= 0")
    if keep is None:
        keep = num_layers // 2
    if not 0 <= keep <= num_layers:
        raise ValueError(f"keep must be in [0, {num_layers}]")
    return range(num_layers - keep, num_layers)


class GuidedQAT:
    """Per-site dispatch for a QAT forward pass: a site (any hashable key, for
    example (layer, "moe_in") or (layer, "kv")) with a rollout record on a
    guided layer gets guided fake quantization; every other site gets
    vanilla FP4 fake quantization. Records are put in by the caller, one per
    site and micro-batch, as the rollout produced them."""

    def __init__(self, num_layers: int, keep: Optional[int] = None, fmt="nvfp4",
                 bits: Optional[int] = None, group_rows: int = 0):
        self.layers = guided_layers(num_layers, keep)
        self.fmt = fmt
        self.bits = bits
        self.group_rows = group_rows
        self.records: Dict[Hashable, Guidance] = {}

    def is_guided(self, layer: int) -> bool:
        return layer in self.layers

    def put(self, site: Hashable, layer: int, g: Guidance) -> None:
        if self.is_guided(layer):
            self.records[(layer, site)] = g

    def clear(self) -> None:
        self.records.clear()

    def __call__(self, x: torch.Tensor, layer: int, site: Hashable = "act") -> torch.Tensor:
        g = self.records.get((layer, site)) if self.is_guided(layer) else None
        if g is None:
            return rtn_fake_quant_ste(x, self.fmt, self.group_rows)
        return guided_fake_quant_ste(x, g, self.bits)

    def guided_sites(self) -> Sequence[Hashable]:
        return sorted(self.records, key=repr)
