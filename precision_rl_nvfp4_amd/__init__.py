"""Rollout-guided FP4 fake quantization for MI355X (gfx950).

Thin torch binding over the C ABI of ``libtrace_fp4.so`` (include/trace_fp4.h).
torch supplies device memory and the current stream; every step of the path
runs in the library's HIP kernels. The calls and their sources in the paper
("TRACE: Rollout-Guided Quantization-Aware Training for FP4 Reinforcement
Learning of MoE Language Models", arXiv 2610.07767):

    quantize_rtn             vanilla FP4 fake quantization (§3.1, Fig. 4(a))
    encode_guidance          rollout-side guidance record (§3.2, §4.2; Algorithm 1)
    decode_guidance          Reconstruct (Algorithm 1)
    guided_fake_quant        rollout-guided rounding (§3.1 "Key Design")
    guided_fake_quant_stats  the same plus the discrepancy sums in one pass
    discrepancy_stats        D_BF16 / D_FP4 sums (§3.1, Fig. 4(b))

Tensors are bf16 [rows, cols] on a gfx950 device, contiguous, with cols a
multiple of the block size (16 for NVFP4, 32 for MXFP4). ``group_rows`` > 0
gives every ``group_rows`` consecutive rows their own FP32 global scale
(NVFP4); 0 means one scale for the whole tensor.
"""

from __future__ import annotations

import math
from typing import NamedTuple, Optional

import torch

from . import _abi
from ._abi import (MISMATCH_COUNTS, MXFP4, NOALLOC_SCRATCH_BYTES, NVFP4, TraceError, load,  # noqa: F401
                   status_str)

MISMATCH_BINS = MISMATCH_COUNTS // 2 - 1   # distances 0..14 per histogram

__all__ = ["NVFP4", "MXFP4", "TraceError", "Quantized", "Guidance", "quantize_rtn",
           "encode_guidance", "encode_guidance_grouped", "decode_guidance", "guided_fake_quant",
           "guided_fake_quant_stats",
           "discrepancy_stats", "stats_workspace", "quant_workspace", "guided_stats_workspace",
           "encode_wait_failures", "encode_guidance_noalloc", "NOALLOC_SCRATCH_BYTES",
           "grouped_workspace", "stream_copy", "stream_mix",
           "derived_metrics", "mismatch_summary", "fmt_id", "BLOCK", "MISMATCH_COUNTS"]

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
    gscale: Optional[torch.Tensor]  # float32 [G, 2] = {S, A} per group (NVFP4) or None
    y: Optional[torch.Tensor]      # bf16 [rows, cols] or None


class Guidance(NamedTuple):
    fmt: int
    bits: int
    guide: torch.Tensor            # uint8 [rows, cols/8] (bits=1) or [rows, cols/2] (bits=4)
    scales: torch.Tensor           # uint8 [rows, cols/B]
    gscale: Optional[torch.Tensor]  # float32 [G, 2] (NVFP4) or None
    y: Optional[torch.Tensor]      # the rollout's own dequantized bf16 output, or None
    group_rows: int = 0
    offsets: Optional[torch.Tensor] = None  # int64 [G + 1] device row offsets (row-offset groups)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _nbytes(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.numel() * t.element_size()


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


def _groups(rows: int, group_rows: int) -> int:
    if group_rows < 0 or (group_rows > 0 and rows % group_rows):
        raise ValueError(f"group_rows={group_rows} must be 0 or divide rows={rows}")
    return rows // group_rows if group_rows > 0 else 1


def _empty(shape, dtype, like: torch.Tensor, out: Optional[torch.Tensor]):
    if out is not None:
        if tuple(out.shape) != tuple(shape) or out.dtype != dtype or not out.is_contiguous():
            raise ValueError(f"output buffer must be contiguous {dtype} {tuple(shape)}")
        return out
    return torch.empty(shape, dtype=dtype, device=like.device)


def _workspace(nbytes: int, device, work: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes < 0:
        raise ValueError("invalid shape")
    if work is not None:
        return work
    if nbytes == 0:
        return None
    return torch.empty((nbytes + 7) // 8, dtype=torch.float64, device=device)


def encode_wait_failures() -> int:
    """Bounded waits of the single-pass encode that gave up on the current
    device since the library was loaded. Each one was recovered exactly (the
    missing maxima were read from the input), so a nonzero count means slower
    calls, not wrong results. Synchronize the encode calls' streams first."""
    import ctypes
    v = ctypes.c_uint64()
    _abi.call("trace_encode_wait_failures", ctypes.byref(v))
    return int(v.value)


def quant_workspace(fmt, rows: int, cols: int, group_rows: int = 0, device="cuda"):
    """Workspace tensor for quantize_rtn / encode_guidance with scales from the amax."""
    n = int(load().trace_quant_workspace_bytes(fmt_id(fmt), rows, cols, group_rows))
    return _workspace(n, device, None)


def grouped_workspace(fmt, rows: int, cols: int, groups: int, device="cuda"):
    """Workspace tensor for the row-offset grouped calls."""
    n = int(load().trace_grouped_workspace_bytes(fmt_id(fmt), rows, cols, groups))
    return _workspace(n, device, None)


def guided_stats_workspace(fmt, rows: int, cols: int, group_rows: int = 0, device="cuda"):
    n = int(load().trace_guided_stats_workspace_bytes(fmt_id(fmt), rows, cols, group_rows))
    return _workspace(n, device, None)


def stats_workspace(n: int, device) -> torch.Tensor:
    nbytes = int(load().trace_stats_workspace_bytes(int(n)))
    return torch.empty(max(nbytes // 8, 2), dtype=torch.float64, device=device)


def _rtn_call(name, x, f, bits, group_rows, gscale, plane_shape, with_y, plane, scales,
              gscale_out, y, work):
    rows, cols = _check_x(x)
    G = _groups(rows, group_rows)
    plane = _empty(plane_shape, torch.uint8, x, plane)
    scales = _empty((rows, cols // BLOCK[f]), torch.uint8, x, scales)
    if f == NVFP4 and gscale is None:
        gscale_out = _empty((G, 2), torch.float32, x, gscale_out)
        need = int(load().trace_quant_workspace_bytes(f, rows, cols, group_rows))
        work = _workspace(need, x.device, work)
    else:
        gscale_out = None
        work = None
    y = _empty((rows, cols), torch.bfloat16, x, y) if with_y else None
    head = [f] if bits is None else [f, int(bits)]
    _abi.call(name, *head, rows, cols, group_rows, _ptr(x), _ptr(gscale), _ptr(plane), _ptr(scales),
              _ptr(gscale_out), _ptr(y), _ptr(work), _nbytes(work), _stream(x))
    return plane, scales, (gscale if gscale is not None else gscale_out), y


def quantize_rtn(x: torch.Tensor, fmt="nvfp4", gscale: Optional[torch.Tensor] = None,
                 with_y: bool = True, group_rows: int = 0, codes=None, scales=None,
                 gscale_out=None, y=None, work=None) -> Quantized:
    """RTN FP4 fake quantization of x with its own scales. For NVFP4 the global
    scale of each group comes from its amax unless ``gscale`` (a device float
    tensor holding S of group g at flat index 2g) is given."""
    f = fmt_id(fmt)
    rows, cols = _check_x(x)
    c, s, g, yy = _rtn_call("quantize_rtn", x, f, None, group_rows, gscale, (rows, cols // 2),
                            with_y, codes, scales, gscale_out, y, work)
    return Quantized(c, s, g, yy)


def encode_guidance(x_rollout: torch.Tensor, fmt="nvfp4", bits: int = 1,
                    gscale: Optional[torch.Tensor] = None, with_y: bool = False,
                    group_rows: int = 0, guide=None, scales=None, gscale_out=None, y=None,
                    work=None) -> Guidance:
    """Rollout side: RTN-quantize and emit the guidance record (bits=1: the
    mantissa-bit plane; 2, 3: the low magnitude bits; 4: the full code plane)
    plus the scales."""
    f = fmt_id(fmt)
    rows, cols = _check_x(x_rollout, "x_rollout")
    if bits not in (1, 2, 3, 4):
        raise ValueError("bits must be 1, 2, 3 or 4")
    gcols = cols * bits // 8
    c, s, g, yy = _rtn_call("encode_guidance", x_rollout, f, bits, group_rows, gscale,
                            (rows, gcols), with_y, guide, scales, gscale_out, y, work)
    return Guidance(f, int(bits), c, s, g, yy, int(group_rows))


def encode_guidance_noalloc(x_rollout: torch.Tensor, fmt="nvfp4", bits: int = 1,
                            gscale: Optional[torch.Tensor] = None, group_rows: int = 0, *,
                            guide: torch.Tensor, scales: torch.Tensor,
                            gscale_out: Optional[torch.Tensor] = None,
                            y: Optional[torch.Tensor] = None) -> Guidance:
    """encode_guidance into caller buffers with no workspace argument: where a
    workspace is needed the library uses its own per-device scratch array (up
    to NOALLOC_SCRATCH_BYTES; larger calls raise). Nothing is allocated, so it
    can run where allocation cannot (e.g. under graph capture). Calls that
    overlap on one device share that array and must be ordered."""
    f = fmt_id(fmt)
    rows, cols = _check_x(x_rollout, "x_rollout")
    if bits not in (1, 2, 3, 4):
        raise ValueError("bits must be 1, 2, 3 or 4")
    G = _groups(rows, group_rows)
    guide = _empty((rows, cols * bits // 8), torch.uint8, x_rollout, guide)
    scales = _empty((rows, cols // BLOCK[f]), torch.uint8, x_rollout, scales)
    if f == NVFP4 and gscale is None:
        if gscale_out is None:
            raise ValueError("gscale_out (float32 [G, 2]) is required when gscale is not given")
        gscale_out = _empty((G, 2), torch.float32, x_rollout, gscale_out)
    else:
        gscale_out = None
    if y is not None:
        y = _empty((rows, cols), torch.bfloat16, x_rollout, y)
    _abi.call("encode_guidance_noalloc", f, int(bits), rows, cols, group_rows, _ptr(x_rollout), _ptr(gscale),
              _ptr(guide), _ptr(scales), _ptr(gscale_out), _ptr(y), _stream(x_rollout))
    return Guidance(f, int(bits), guide, scales, gscale if gscale is not None else gscale_out, y,
                    int(group_rows))


def _check_offsets(offsets: torch.Tensor, x: torch.Tensor) -> int:
    if (offsets.dtype != torch.int64 or offsets.dim() != 1 or offsets.numel() < 2
            or not offsets.is_contiguous() or offsets.device != x.device):
        raise ValueError("row offsets must be a contiguous int64 [G + 1] tensor on x's device")
    return offsets.numel() - 1


def encode_guidance_grouped(x_rollout: torch.Tensor, offsets: torch.Tensor, fmt="nvfp4", bits: int = 1,
                            with_y: bool = False, guide=None, scales=None, gscale_out=None, y=None,
                            work=None) -> Guidance:
    """encode_guidance with one global scale per row-offset group (e.g. per
    expert of a grouped MoE input): group g is rows [offsets[g], offsets[g+1])."""
    f = fmt_id(fmt)
    rows, cols = _check_x(x_rollout, "x_rollout")
    G = _check_offsets(offsets, x_rollout)
    if bits not in (1, 2, 3, 4):
        raise ValueError("bits must be 1, 2, 3 or 4")
    guide = _empty((rows, cols * bits // 8), torch.uint8, x_rollout, guide)
    scales = _empty((rows, cols // BLOCK[f]), torch.uint8, x_rollout, scales)
    gscale_out = _empty((G, 2), torch.float32, x_rollout, gscale_out) if f == NVFP4 else None
    y = _empty((rows, cols), torch.bfloat16, x_rollout, y) if with_y else None
    need = int(load().trace_grouped_workspace_bytes(f, rows, cols, G))
    work = _workspace(need, x_rollout.device, work)
    _abi.call("encode_guidance_grouped", f, int(bits), rows, cols, G, _ptr(offsets), _ptr(x_rollout),
              _ptr(guide), _ptr(scales), _ptr(gscale_out), _ptr(y), _ptr(work), _nbytes(work),
              _stream(x_rollout))
    return Guidance(f, int(bits), guide, scales, gscale_out, y, 0, offsets)


def decode_guidance(x_train: torch.Tensor, g: Guidance, ref_codes=None) -> torch.Tensor:
    """Reconstruct the compact rollout reference codes (records of 1..3 bits)."""
    if g.bits not in (1, 2, 3):
        raise ValueError("decode_guidance takes a record of 1, 2 or 3 bits")
    if g.offsets is not None:
        raise ValueError("decode_guidance takes equal groups")
    rows, cols = _check_x(x_train, "x_train")
    ref_codes = _empty((rows, cols // 2), torch.uint8, x_train, ref_codes)
    _abi.call("decode_guidance", g.fmt, g.bits, rows, cols, g.group_rows, _ptr(x_train), _ptr(g.guide),
              _ptr(g.scales), _ptr(g.gscale), _ptr(ref_codes), _stream(x_train))
    return ref_codes


def _guided_common(x_train, g, bits, with_codes, y, codes):
    b = g.bits if bits is None else int(bits)
    if b not in (0, g.bits):
        raise ValueError(f"record holds bits={g.bits}, asked for bits={b}")
    rows, cols = _check_x(x_train, "x_train")
    y = _empty((rows, cols), torch.bfloat16, x_train, y)
    codes = _empty((rows, cols // 2), torch.uint8, x_train, codes) if with_codes else None
    guide = None if b == 0 else g.guide
    return b, rows, cols, y, codes, guide


def guided_fake_quant(x_train: torch.Tensor, g: Guidance, bits: Optional[int] = None,
                      with_codes: bool = False, y=None, codes=None, work=None):
    """Training side: rollout-guided rounding under the rollout scales.
    ``bits`` defaults to the record's (1..4); 0 gives RTN under the rollout
    scales. Returns (y, codes or None)."""
    b, rows, cols, y, codes, guide = _guided_common(x_train, g, bits, with_codes, y, codes)
    if g.offsets is not None:   # row-offset groups
        G = _check_offsets(g.offsets, x_train)
        need = int(load().trace_grouped_workspace_bytes(g.fmt, rows, cols, G))
        work = _workspace(need, x_train.device, work)
        _abi.call("guided_fake_quant_grouped", g.fmt, b, rows, cols, G, _ptr(g.offsets), _ptr(x_train),
                  _ptr(guide), _ptr(g.scales), _ptr(g.gscale), _ptr(y), _ptr(codes), _ptr(work),
                  _nbytes(work), _stream(x_train))
        return y, codes
    _abi.call("guided_fake_quant", g.fmt, b, rows, cols, g.group_rows, _ptr(x_train), _ptr(guide),
              _ptr(g.scales), _ptr(g.gscale), _ptr(y), _ptr(codes), _stream(x_train))
    return y, codes


def guided_fake_quant_stats(x_train: torch.Tensor, x_rollout: torch.Tensor, g: Guidance,
                            bits: Optional[int] = None, with_codes: bool = False,
                            acc: Optional[torch.Tensor] = None, accumulate: bool = False,
                            y=None, codes=None, work=None, mismatch: bool = False,
                            counts: Optional[torch.Tensor] = None):
    """guided_fake_quant plus {SB, SF, n} against the rollout (whose RTN output
    under the record's scales is recomputed from x_rollout). Returns
    (y, codes or None, acc float64[3]); with mismatch=True (or a counts
    tensor) also the int64[32] mismatch diagnostics, as a fourth element
    (layout in mismatch_summary)."""
    if g.offsets is not None:
        raise ValueError("guided_fake_quant_stats takes equal groups; for row-offset groups use "
                         "guided_fake_quant and discrepancy_stats")
    b, rows, cols, y, codes, guide = _guided_common(x_train, g, bits, with_codes, y, codes)
    _check_x(x_rollout, "x_rollout")
    if tuple(x_rollout.shape) != (rows, cols):
        raise ValueError("x_rollout must have x_train's shape")
    if acc is None:
        if accumulate:
            raise ValueError("accumulate=True needs an acc tensor")
        acc = torch.empty(3, dtype=torch.float64, device=x_train.device)
    want_counts = mismatch or counts is not None
    if want_counts:
        if counts is None:
            if accumulate:
                raise ValueError("accumulate=True needs a counts tensor")
            counts = torch.empty(MISMATCH_COUNTS, dtype=torch.int64, device=x_train.device)
        elif (counts.dtype != torch.int64 or counts.numel() != MISMATCH_COUNTS
              or not counts.is_contiguous() or counts.device != x_train.device):
            raise ValueError(f"counts must be a contiguous int64[{MISMATCH_COUNTS}] on x_train's device")
    need = int(load().trace_guided_stats_workspace_bytes(g.fmt, rows, cols, g.group_rows))
    work = _workspace(need, x_train.device, work)
    _abi.call("guided_fake_quant_stats", g.fmt, b, rows, cols, g.group_rows, _ptr(x_train),
              _ptr(x_rollout), _ptr(guide), _ptr(g.scales), _ptr(g.gscale), _ptr(y), _ptr(codes),
              _ptr(acc), _ptr(counts) if want_counts else None, 1 if accumulate else 0, _ptr(work),
              _nbytes(work), _stream(x_train))
    if want_counts:
        return y, codes, acc, counts
    return y, codes, acc


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
              1 if accumulate else 0, _ptr(work), _nbytes(work), _stream(x_t))
    return acc


def _stream_bytes(*ts) -> int:
    n = ts[0].numel() * ts[0].element_size()
    for t in ts:
        if not t.is_contiguous() or t.device.type != "cuda" or t.numel() * t.element_size() != n:
            raise ValueError("stream references take contiguous device tensors of one byte size")
    return n


def stream_copy(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """Measurement reference (no step of the method): dst = src as a plain
    stream with the path kernels' access policy."""
    n = _stream_bytes(src, dst)
    _abi.call("trace_stream_copy", _ptr(src), _ptr(dst), n, _stream(src))
    return dst


def stream_mix(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor) -> torch.Tensor:
    """Measurement reference (no step of the method): out = a XOR b, bytewise,
    two streams read and one written (the fused guided pass's mix)."""
    n = _stream_bytes(a, b, out)
    _abi.call("trace_stream_mix", _ptr(a), _ptr(b), _ptr(out), n, _stream(a))
    return out


def mismatch_summary(counts) -> dict:
    """Host-side view of guided_fake_quant_stats' mismatch counts (§3.2
    "Key Design", Fig. 6). counts[0..14]: elements whose guided code is
    0..14 grid positions from the rollout code; counts[15..29]: the same for
    RTN under the rollout scales; counts[30] / [31]: guidance moved the
    magnitude up / down relative to RTN."""
    c = [int(v) for v in (counts.tolist() if hasattr(counts, "tolist") else counts)]
    nb = MISMATCH_BINS
    guided, rtn = c[:nb], c[nb:2 * nb]
    n = sum(guided)
    rtn_mis = n - rtn[0]
    guided_mis = n - guided[0]
    return {"n": n,
            "rtn_mismatch": rtn_mis, "rtn_mismatch_rate": rtn_mis / n if n else math.nan,
            "rtn_adjacent_fraction": rtn[1] / rtn_mis if rtn_mis else math.nan,
            "guided_mismatch": guided_mis, "guided_mismatch_rate": guided_mis / n if n else math.nan,
            "guided_adjacent_fraction": guided[1] / guided_mis if guided_mis else math.nan,
            "moved_up": c[2 * nb], "moved_down": c[2 * nb + 1],
            "guided_hist": guided, "rtn_hist": rtn}


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
