"""Record path bindings: the pinned-host ring that takes finished guidance
records off the GPU, and the page gather of a paged record (include/trace_fp4.h,
"Record path"). Argument marshalling only; the copies and the gather run in
libtrace_fp4.so."""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import _abi

__all__ = ["RecordRing", "gather_pages"]


def _stream_of(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


class RecordRing:
    """`slots` pinned host buffers of `slot_bytes` each, filled in ring order
    by device-to-host copies on the ring's own stream.

    The copies of a push run later, on the ring's stream, so the ring keeps a
    reference to the pushed tensors until the slot's copies are known to be
    done (wait, ready returning True, release or close): a caller may drop
    them, or reuse their memory through torch's caching allocator, right
    after push."""

    def __init__(self, slot_bytes: int, slots: int):
        self._lib = _abi.load()
        h = ctypes.c_void_p()
        _abi.call("trace_ring_create", int(slot_bytes), int(slots), ctypes.byref(h))
        self._h = h
        self.slot_bytes = int(slot_bytes)
        self.slots = int(slots)
        self._held = [[] for _ in range(self.slots)]   # sources of each slot's copies in flight

    def push(self, tensors: Sequence[torch.Tensor], stream: Optional[int] = None) -> int:
        """Queue copies of the (contiguous, device) tensors, back to back, into
        the next slot, after the work already enqueued on `stream` (default:
        torch's current stream of the first tensor). Returns the slot. The
        tensors are kept alive by the ring until the copies are done."""
        if not tensors:
            raise ValueError("push needs at least one tensor")
        for t in tensors:
            if not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError("push takes contiguous device tensors")
        n = len(tensors)
        srcs = (ctypes.c_void_p * n)(*[t.data_ptr() for t in tensors])
        sizes = (ctypes.c_int64 * n)(*[t.numel() * t.element_size() for t in tensors])
        slot = ctypes.c_int32()
        s = _stream_of(tensors[0]) if stream is None else stream
        _abi.call("trace_ring_push", self._h, srcs, sizes, n, s, ctypes.byref(slot))
        self._held[slot.value] = list(tensors)
        return slot.value

    def wait(self, slot: int) -> None:
        _abi.call("trace_ring_wait", self._h, int(slot))
        self._held[int(slot)] = []

    def ready(self, slot: int) -> bool:
        r = self._lib.trace_ring_query(self._h, int(slot))
        if r < 0:
            raise _abi.TraceError("trace_ring_query", r)
        if r == 1:
            self._held[int(slot)] = []
        return r == 1

    def view(self, slot: int) -> np.ndarray:
        """The bytes of a DONE slot as a uint8 array over the pinned memory
        (valid until the slot is released)."""
        nbytes = ctypes.c_int64()
        p = self._lib.trace_ring_slot(self._h, int(slot), ctypes.byref(nbytes))
        if not p:
            raise RuntimeError(f"slot {slot} is not done")
        if nbytes.value == 0:
            return np.zeros(0, np.uint8)
        return np.ctypeslib.as_array((ctypes.c_uint8 * nbytes.value).from_address(p))

    def release(self, slot: int) -> None:
        _abi.call("trace_ring_release", self._h, int(slot))
        self._held[int(slot)] = []

    def close(self) -> None:
        if self._h is not None:
            _abi.call("trace_ring_destroy", self._h)   # waits for the ring's copies
            self._h = None
            self._held = [[] for _ in range(self.slots)]

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def gather_pages(pool: torch.Tensor, page_bytes: int, page_ids: torch.Tensor,
                 out: Optional[torch.Tensor] = None, bad: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[i] = page page_ids[i] of `pool` (uint8, whole pages); ids outside
    the pool give zero pages and are counted into `bad` (uint32[1]) if given."""
    if pool.dtype != torch.uint8 or not pool.is_contiguous() or pool.device.type != "cuda":
        raise ValueError("pool must be a contiguous uint8 device tensor")
    if page_bytes <= 0 or pool.numel() % page_bytes:
        raise ValueError("pool must hold whole pages")
    if page_ids.dtype != torch.int32 or not page_ids.is_contiguous() or page_ids.device != pool.device:
        raise ValueError("page_ids must be contiguous int32 on the pool's device")
    n = page_ids.numel()
    if out is None:
        out = torch.empty(n * page_bytes, dtype=torch.uint8, device=pool.device)
    elif out.dtype != torch.uint8 or not out.is_contiguous() or out.numel() != n * page_bytes:
        raise ValueError("out must be contiguous uint8 of n * page_bytes")
    if bad is not None and (bad.dtype != torch.uint32 or bad.numel() != 1):
        raise ValueError("bad must be a uint32[1] device tensor")
    _abi.call("trace_gather_pages", pool.data_ptr(), pool.numel() // page_bytes, int(page_bytes),
              page_ids.data_ptr(), n, out.data_ptr(), None if bad is None else bad.data_ptr(),
              _stream_of(pool))
    return out
