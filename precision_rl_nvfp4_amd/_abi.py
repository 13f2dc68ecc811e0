"""ctypes view of the C ABI in include/trace_fp4.h.

Loading fails loudly when the library has not been built; there is no
fallback implementation anywhere in the package.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtrace_fp4.so")

OK, EINVAL, ESHAPE, EALIGN, EALIAS, EDEVICE, ELAUNCH, EBUSY = 0, -1, -2, -3, -4, -5, -6, -7
NVFP4, MXFP4 = 0, 1
ABI_VERSION = 9
MISMATCH_COUNTS = 32
NOALLOC_SCRATCH_BYTES = 4 << 20

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p

# name -> (restype, argtypes); pointers are passed as integers (device addresses).
SIGNATURES = {
    "trace_abi_version": (_int, []),
    "trace_status_str": (ctypes.c_char_p, [_int]),
    "trace_set_encode_batch": (_i64, [_i64]),
    "trace_set_wait_limit": (_i64, [_i64]),
    "trace_encode_wait_failures": (_int, [ctypes.POINTER(ctypes.c_uint64)]),
    "trace_quant_workspace_bytes": (_i64, [_int, _i64, _i64, _i64]),
    "trace_guided_stats_workspace_bytes": (_i64, [_int, _i64, _i64, _i64]),
    "trace_stats_workspace_bytes": (_i64, [_i64]),
    # fmt, rows, cols, group_rows, x, gscale_in, codes, scales, gscale_out, y, work, work_bytes, stream
    "quantize_rtn": (_int, [_int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    # fmt, bits, rows, cols, group_rows, x_r, gscale_in, guide, scales, gscale_out, y_r, work, work_bytes, stream
    "encode_guidance": (_int, [_int, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    # fmt, bits, rows, cols, group_rows, x_r, gscale_in, guide, scales, gscale_out, y_r, stream
    "encode_guidance_noalloc": (_int, [_int, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    # fmt, bits, rows, cols, group_rows, x_t, guide, scales, gscale, ref_codes, stream
    "decode_guidance": (_int, [_int, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    # fmt, bits, rows, cols, group_rows, x_t, guide, scales, gscale, y, codes, stream
    "guided_fake_quant": (_int, [_int, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    # fmt, bits, rows, cols, group_rows, x_t, x_r, guide, scales, gscale, y, codes, acc3, counts,
    # accumulate, work, work_bytes, stream
    "guided_fake_quant_stats": (_int, [_int, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _int, _vp, _i64, _vp]),
    # n, x_t, x_r, y_t, y_r, acc3, accumulate, work, work_bytes, stream
    "discrepancy_stats": (_int, [_i64, _vp, _vp, _vp, _vp, _vp, _int, _vp, _i64, _vp]),
    # row-offset groups: fmt, rows, cols, groups
    "trace_grouped_workspace_bytes": (_i64, [_int, _i64, _i64, _i64]),
    # fmt, bits, rows, cols, groups, offsets, x_r, guide, scales, gscale_out, y_r, work, work_bytes, stream
    "encode_guidance_grouped": (_int, [_int, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _i64, _vp]),
    # fmt, bits, rows, cols, groups, offsets, x_t, guide, scales, gscale, y, codes, work, work_bytes, stream
    "guided_fake_quant_grouped": (_int, [_int, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _vp, _i64, _vp]),
    # record path: slot_bytes, slots, &ring / ring / ring, srcs, bytes, n, stream, &slot / ...
    "trace_ring_create": (_int, [_i64, ctypes.c_int32, ctypes.POINTER(_vp)]),
    "trace_ring_destroy": (_int, [_vp]),
    "trace_ring_push": (_int, [_vp, ctypes.POINTER(_vp), ctypes.POINTER(_i64), ctypes.c_int32, _vp,
                               ctypes.POINTER(ctypes.c_int32)]),
    "trace_ring_wait": (_int, [_vp, ctypes.c_int32]),
    "trace_ring_query": (_int, [_vp, ctypes.c_int32]),
    "trace_ring_slot": (_vp, [_vp, ctypes.c_int32, ctypes.POINTER(_i64)]),
    "trace_ring_release": (_int, [_vp, ctypes.c_int32]),
    # pool, pool_pages, page_bytes, page_ids, n, out, bad_ids, stream
    "trace_gather_pages": (_int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
    "trace_stream_copy": (_int, [_vp, _vp, _i64, _vp]),
    "trace_stream_mix": (_int, [_vp, _vp, _vp, _i64, _vp]),
}

_lib = None


class TraceError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call} failed: {status_str(status)} ({status})")


def load() -> ctypes.CDLL:
    """The loaded library (loaded once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not built: {LIB_PATH} is missing "
                "(run `python -m precision_rl_nvfp4_amd.build` or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.trace_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {lib.trace_abi_version()}, the binding "
                               f"expects {ABI_VERSION}: rebuild the library")
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load().trace_status_str(int(status)).decode()


def call(name: str, *args) -> None:
    """Invoke an entry point and raise TraceError on a non-zero status."""
    st = getattr(load(), name)(*args)
    if st != OK:
        raise TraceError(name, st)
