"""ctypes view of the C ABI in include/trace_fp4.h.

Loading fails loudly when the library has not been built; there is no
fallback implementation anywhere in the package.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtrace_fp4.so")

OK, EINVAL, ESHAPE, EALIGN, EALIAS, EDEVICE, ELAUNCH = 0, -1, -2, -3, -4, -5, -6
NVFP4, MXFP4 = 0, 1

_i64 = ctypes.c_int64
_int = ctypes.c_int
_vp = ctypes.c_void_p

# name -> (restype, argtypes); pointers are passed as integers (device addresses).
SIGNATURES = {
    "trace_abi_version": (_int, []),
    "trace_status_str": (ctypes.c_char_p, [_int]),
    "quantize_rtn": (_int, [_int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "encode_guidance": (_int, [_int, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "decode_guidance": (_int, [_int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "guided_fake_quant": (_int, [_int, _int, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "discrepancy_stats": (_int, [_i64, _vp, _vp, _vp, _vp, _vp, _int, _vp, _i64, _vp]),
    "trace_stats_workspace_bytes": (_i64, [_i64]),
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
        _lib = lib
    return _lib


def status_str(status: int) -> str:
    return load().trace_status_str(int(status)).decode()


def call(name: str, *args) -> None:
    """Invoke an entry point and raise TraceError on a non-zero status."""
    st = getattr(load(), name)(*args)
    if st != OK:
        raise TraceError(name, st)
