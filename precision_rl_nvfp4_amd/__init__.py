"""Rollout-guided FP4 fake quantization for MI355X (gfx950).

Thin torch binding over the C ABI of ``libtrace_fp4.so`` (include/trace_fp4.h).
torch supplies device memory and the current stream; every step of the path
runs in the library's HIP kernels. The calls and their sources in the paper
("TRACE: Rollout-Guided Quantization-Aware Training for FP4 Reinforcement
Learning of MoE Language Models", arXiv 2610.07767):

    quantize_rtn        vanilla FP4 fake quantization (§3.1, Fig. 4(a))
    encode_guidance     rollout-side guidance record (§3.2, §4.2; Algorithm 1)
    decode_guidance     Reconstruct (Algorithm 1)
    guided_fake_quant   rollout-guided rounding (§3.1 "Key Design")
    discrepancy_stats   D_BF16 / D_FP4 sums (§3.1, Fig. 4(b))

Tensors are bf16 [rows, cols] on a gfx950 device, contiguous, with cols a
multiple of the block size (16 for NVFP4, 32 for MXFP4).
"""

from __future__ import annotations

import math
from typing import NamedTuple, Optional

import torch

from . import _abi
from ._abi import MXFP4, NVFP4, TraceError, load, status_str  # noqa: F401

__all__ = ["NVFP4", "MXFP4", "TraceError", "Quantized", "Guidance", "quantize_rtn",
           "encode_guidance", "decode_guidance", "guided_fake_quant", "discrepancy_stats",
           "stats_workspace", "derived_metrics", "fmt_id", "BLOCK"]

BLOCK = {NVFP4: 16, MXFP4: 32}


def fmt_id(fmt) -> int:
    if fmt in (NVFP4, "nvfp4", "NVFP4"):
        return NVFP4
    if fmt in (MXFP4, "mxfp4", "MXFP4"):
        return MXFP4
    raise ValueError(f"unknown format {fmt!r}")


class Quantized(NamedTuple):
    codes: torch.Tensor            # uint8 [rows, cols/2]
    scales: torch.Tensor           # uint8 [rows, cols/B]
    gscale: Optional[torch.Tensor]  # float32 [2] = {S, A} (NVFP4) or None
    y: Optional[torch.Tensor]      # bf16 [rows, cols] or None


class Guidance(NamedTuple):
    fmt: int
    bits: int
    guide: torch.Tensor            # uint8 [rows, cols/8] (bits=1) or [rows, cols/2] (bits=4)
    scales: torch.Tensor           # uint8 [rows, cols/B]
    gscale: Optional[torch.Tensor]  # float32 [2] (NVFP4) or None
    y: Optional[torch.Tensor]      # the rollout's own dequantized bf16 output, or None


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_x(x: torch.Tensor, name: str = "x") -> tuple[int, int]:
    if x.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {x.dtype}")
    if x.dim() != 2:
        raise ValueError(f"{name} must be 2-D [rows, cols]")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if x.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    return x.shape[0], x.shape[1]


def _empty(shape, dtype, like: torch.Tensor, out: Optional[torch.Tensor]):
    if out is not None:
        if tuple(out.shape) != tuple(shape) or out.dtype != dtype or not out.is_contiguous():
            raise ValueError(f"output buffer must be contiguous {dtype} {tuple(shape)}")
        return out
    return torch.empty(shape, dtype=dtype, device=like.device)


def quantize_rtn(x: torch.Tensor, fmt="nvfp4", gscale: Optional[torch.Tensor] = None,
                 with_y: bool = True, codes=None, scales=None, gscale_out=None, y=None) -> Quantized:
    """RTN FP4 fake quantization of x with its own scales. For NVFP4 the global
    scale comes from the tensor amax unless ``gscale`` (a device float tensor
    whose [0] is S) is given."""
    f = fmt_id(fmt)
    rows, cols = _check_x(x)
    codes = _empty((rows, cols // 2), torch.uint8, x, codes)
    scales = _empty((rows, cols // BLOCK[f]), torch.uint8, x, scales)
    if f == NVFP4 and gscale is None:
        gscale_out = _empty((2,), torch.float32, x, gscale_out)
    else:
        gscale_out = None
    y = _empty((rows, cols), torch.bfloat16, x, y) if with_y else None
    _abi.call("quantize_rtn", f, rows, cols, _ptr(x), _ptr(gscale), _ptr(codes), _ptr(scales),
              _ptr(gscale_out), _ptr(y), _stream(x))
    return Quantized(codes, scales, gscale if gscale is not None else gscale_out, y)


def encode_guidance(x_rollout: torch.Tensor, fmt="nvfp4", bits: int = 1,
                    gscale: Optional[torch.Tensor] = None, with_y: bool = False,
                    guide=None, scales=None, gscale_out=None, y=None) -> Guidance:
    """Rollout side: RTN-quantize and emit the guidance record (bits=1: the
    mantissa-bit plane; bits=4: the full code plane) plus the scales."""
    f = fmt_id(fmt)
    rows, cols = _check_x(x_rollout, "x_rollout")
    gcols = cols // 8 if bits == 1 else cols // 2
    guide = _empty((rows, gcols), torch.uint8, x_rollout, guide)
    scales = _empty((rows, cols // BLOCK[f]), torch.uint8, x_rollout, scales)
    if f == NVFP4 and gscale is None:
        gscale_out = _empty((2,), torch.float32, x_rollout, gscale_out)
    else:
        gscale_out = None
    y = _empty((rows, cols), torch.bfloat16, x_rollout, y) if with_y else None
    _abi.call("encode_guidance", f, int(bits), rows, cols, _ptr(x_rollout), _ptr(gscale),
              _ptr(guide), _ptr(scales), _ptr(gscale_out), _ptr(y), _stream(x_rollout))
    return Guidance(f, int(bits), guide, scales, gscale if gscale is not None else gscale_out, y)


def decode_guidance(x_train: torch.Tensor, g: Guidance, ref_codes=None) -> torch.Tensor:
    """Reconstruct the compact rollout reference codes (bits=1 records only)."""
    if g.bits != 1:
        raise ValueError("decode_guidance takes a bits=1 record")
    rows, cols = _check_x(x_train, "x_train")
    ref_codes = _empty((rows, cols // 2), torch.uint8, x_train, ref_codes)
    _abi.call("decode_guidance", g.fmt, rows, cols, _ptr(x_train), _ptr(g.guide), _ptr(g.scales),
              _ptr(g.gscale), _ptr(ref_codes), _stream(x_train))
    return ref_codes


def guided_fake_quant(x_train: torch.Tensor, g: Guidance, bits: Optional[int] = None,
                      with_codes: bool = False, y=None, codes=None):
    """Training side: rollout-guided rounding under the rollout scales.
    ``bits`` defaults to the record's (1 or 4); 0 gives RTN under the rollout
    scales. Returns (y, codes or None)."""
    b = g.bits if bits is None else int(bits)
    rows, cols = _check_x(x_train, "x_train")
    y = _empty((rows, cols), torch.bfloat16, x_train, y)
    codes = _empty((rows, cols // 2), torch.uint8, x_train, codes) if with_codes else None
    guide = None if b == 0 else g.guide
    if b not in (0, g.bits):
        raise ValueError(f"record holds bits={g.bits}, asked for bits={b}")
    _abi.call("guided_fake_quant", g.fmt, b, rows, cols, _ptr(x_train), _ptr(guide), _ptr(g.scales),
              _ptr(g.gscale), _ptr(y), _ptr(codes), _stream(x_train))
    return y, codes


def stats_workspace(n: int, device) -> torch.Tensor:
    nbytes = int(load().trace_stats_workspace_bytes(int(n)))
    return torch.empty(max(nbytes // 8, 2), dtype=torch.float64, device=device)


def discrepancy_stats(x_t, x_r, y_t, y_r, acc: Optional[torch.Tensor] = None,
                      accumulate: bool = False, work: Optional[torch.Tensor] = None) -> torch.Tensor:
    """{SB, SF, n} as a float64 [3] device tensor; accumulate=True adds to acc."""
    n = x_t.numel()
    for t in (x_t, x_r, y_t, y_r):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or t.numel() != n:
            raise ValueError("discrepancy_stats takes four contiguous bf16 tensors of one size")
    if acc is None:
        if accumulate:
            raise ValueError("accumulate=True needs an acc tensor")
        acc = torch.empty(3, dtype=torch.float64, device=x_t.device)
    if work is None:
        work = stats_workspace(n, x_t.device)
    _abi.call("discrepancy_stats", n, _ptr(x_t), _ptr(x_r), _ptr(y_t), _ptr(y_r), _ptr(acc),
              1 if accumulate else 0, _ptr(work), work.numel() * 8, _stream(x_t))
    return acc


def derived_metrics(acc3) -> dict:
    """D_BF16 = SB/n, D_FP4 = SF/n, relative excess (SF - SB)/SB (+inf when
    SB = 0 < SF, NaN for 0/0) and D_act = sqrt(SF) (§3.1, Eq. 1 and Fig. 4(b))."""
    sb, sf, n = (float(v) for v in acc3)
    if sb > 0:
        rel = (sf - sb) / sb
    else:
        rel = math.inf if sf > 0 else math.nan
    return {"SB": sb, "SF": sf, "n": n, "D_BF16": sb / n if n else math.nan,
            "D_FP4": sf / n if n else math.nan, "rel_excess": rel, "D_act": math.sqrt(sf)}
