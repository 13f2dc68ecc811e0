"""The C-ABI library loads without a GPU, exports every call the header
declares, and rejects bad arguments on the host before any HIP call.

No test here may reach a kernel launch: every call below fails validation,
except the EDEVICE check, which only runs when no GPU is visible.
"""

import ctypes
import os
import re

import pytest
import torch

from precision_rl_nvfp4_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "trace_fp4.h")

A = 0x100000            # a fake, 16-byte-aligned "device" address; never dereferenced
B = 0x200000
C = 0x300000
D = 0x400000
E = 0x500000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)) - {"if"}


@pytest.fixture(scope="module")
def lib():
    return _abi.load()


def test_library_builds_are_present():
    assert os.path.exists(_abi.LIB_PATH), "run __graft_entry__.build() first"


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"quantize_rtn", "encode_guidance", "decode_guidance", "guided_fake_quant",
            "discrepancy_stats", "trace_abi_version", "trace_status_str",
            "trace_stats_workspace_bytes"} <= names
    raw = ctypes.CDLL(_abi.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(_abi.SIGNATURES) == names


def test_version_and_status_strings(lib):
    assert lib.trace_abi_version() == _abi.ABI_VERSION == 9
    for code, name in [(0, "TRACE_OK"), (-1, "TRACE_EINVAL"), (-2, "TRACE_ESHAPE"),
                       (-3, "TRACE_EALIGN"), (-4, "TRACE_EALIAS"), (-5, "TRACE_EDEVICE"),
                       (-6, "TRACE_ELAUNCH"), (-7, "TRACE_EBUSY"), (7, "unknown status")]:
        assert _abi.status_str(code) == name


def test_encode_batch_setting(lib):
    assert lib.trace_set_encode_batch(3) == 0
    assert lib.trace_set_encode_batch(0) == 3
    assert lib.trace_set_encode_batch(-1) == _abi.EINVAL
    assert lib.trace_set_encode_batch(0) == 0


def test_noalloc_encode_limits(lib):
    """encode_guidance_noalloc: its scratch holds 512 groups' amax workspace
    (8192 bytes each); more is ESHAPE before any device use, at most reaches
    the device check. Argument errors as encode_guidance."""
    assert _abi.NOALLOC_SCRATCH_BYTES == 4 << 20
    f = lib.encode_guidance_noalloc
    # rows of 48 columns, one group per row (6 units: not packed, needs the workspace)
    assert lib.trace_quant_workspace_bytes(0, 512, 48, 1) == _abi.NOALLOC_SCRATCH_BYTES
    assert f(0, 1, 513, 48, 1, A, None, B, C, D, None, None) == _abi.ESHAPE
    assert f(0, 1, 512, 48, 1, A, None, B, C, D, None, None) == _abi.EDEVICE
    # the limit only counts the workspace: S supplied, packed groups, MXFP4 need none
    assert f(0, 1, 4096, 48, 1, A, E, B, C, None, None, None) == _abi.EDEVICE
    assert f(0, 1, 4096, 64, 1, A, None, B, C, D, None, None) == _abi.EDEVICE
    assert f(1, 1, 4096, 64, 0, A, None, B, C, None, None, None) == _abi.EDEVICE
    assert f(0, 5, 4, 32, 0, A, None, B, C, D, None, None) == _abi.EINVAL
    assert f(0, 1, 4, 32, 0, A, E, B, C, D, None, None) == _abi.EINVAL      # gscale_in and out
    assert f(0, 1, 4, 32, 0, A + 8, None, B, C, D, None, None) == _abi.EALIGN
    assert f(0, 1, 4, 32, 0, A, None, B, C, A + 4, None, None) == _abi.EALIAS


def test_wait_failure_query_without_a_device(lib):
    """The give-up count needs a gfx950 device; a NULL output is rejected first."""
    assert lib.trace_encode_wait_failures(None) == _abi.EINVAL
    v = ctypes.c_uint64(7)
    assert lib.trace_encode_wait_failures(ctypes.byref(v)) == _abi.EDEVICE
    assert v.value == 7


def test_wait_limit_setting(lib):
    assert lib.trace_set_wait_limit(5) == 0
    assert lib.trace_set_wait_limit(0) == 5
    assert lib.trace_set_wait_limit(-1) == _abi.EINVAL
    assert lib.trace_set_wait_limit(1 << 31) == _abi.EINVAL
    assert lib.trace_set_wait_limit(0) == 0


TILE = 2048   # units (8 bf16 each) of a workgroup tile of the quantize and two-pass kernels
GTILE = 1024  # units of a tile of guided rounding and the fused statistics


def test_workspace_sizes(lib):
    assert lib.trace_stats_workspace_bytes(0) == 16
    assert lib.trace_stats_workspace_bytes(8192 * 2048) == 16 * 1024
    assert lib.trace_stats_workspace_bytes(-1) == 0
    # per global-scale group 1024 uint32 partial (or tile) maxima + 16 published
    # S words on their own 256-byte lines (1024 words)
    qwb = lambda G: 8192 * G  # noqa: E731
    assert lib.trace_quant_workspace_bytes(0, 4, 32, 0) == qwb(1) == 8192
    assert lib.trace_quant_workspace_bytes(0, 17 * 8192, 2048, 8192) == qwb(17)
    assert lib.trace_quant_workspace_bytes(1, 4, 32, 0) == 0            # MXFP4: no amax pass
    assert lib.trace_quant_workspace_bytes(0, 5, 32, 2) == -1           # 2 does not divide 5
    assert lib.trace_quant_workspace_bytes(3, 4, 32, 0) == -1           # bad format
    # two float64 partial sums per workgroup tile of GTILE units, plus 64 pairs for
    # the first level of the reduction
    # packed groups (power-of-two units below a tile, G > 1) need no amax workspace
    assert lib.trace_quant_workspace_bytes(0, 8, 32, 4) == 0           # 2 groups of 16 units
    assert lib.trace_quant_workspace_bytes(0, 139264, 2048, 1) == 0    # per-token scales
    assert lib.trace_quant_workspace_bytes(0, 6, 32, 3) == qwb(2)      # 12 units: not a power of two
    assert lib.trace_quant_workspace_bytes(0, 16, 2048, 8) == qwb(2)   # 2048 units: whole tiles
    assert lib.trace_quant_workspace_bytes(1, 16, 2048, 8) == 0
    # per-token: 139264 rows x 256 units packed GTILE / 256 to a tile
    t = 139264 * 256 // GTILE
    assert lib.trace_guided_stats_workspace_bytes(0, 139264, 2048, 1) == 16 * (t + 64) + 128 * t
    # MXFP4 groups merge into one tensor: 4 groups of 300 units -> ceil(1200 / GTILE) tiles
    t = (1200 + GTILE - 1) // GTILE
    assert lib.trace_guided_stats_workspace_bytes(1, 4 * 75, 32, 75) == 16 * (t + 64) + 128 * t
    # 16 bytes of sums per tile + 64 second-level pairs, 32 uint32 counts per tile
    assert lib.trace_guided_stats_workspace_bytes(0, 4, 32, 0) == 16 * (1 + 64) + 128
    t = 17 * (8192 * 256 // GTILE)
    assert lib.trace_guided_stats_workspace_bytes(0, 17 * 8192, 2048, 8192) == 16 * (t + 64) + 128 * t
    assert lib.trace_guided_stats_workspace_bytes(0, 4, 24, 0) == -1    # cols % 16


W = 0x600000            # a fake workspace address
WB = 8192               # quantize workspace bytes for one group


# quantize_rtn(fmt, rows, cols, group_rows, x, gin, codes, scales, gout, y, work, work_bytes, stream)
@pytest.mark.parametrize("args,status", [
    ((2, 4, 32, 0, A, None, B, C, D, None, W, WB, None), _abi.EINVAL),          # bad fmt
    ((0, 4, 24, 0, A, None, B, C, D, None, W, WB, None), _abi.ESHAPE),          # cols % 16
    ((1, 4, 48, 0, A, None, B, C, None, None, None, 0, None), _abi.ESHAPE),     # cols % 32
    ((0, -1, 32, 0, A, None, B, C, D, None, W, WB, None), _abi.ESHAPE),         # negative rows
    ((0, 4, 32, -2, A, None, B, C, D, None, W, WB, None), _abi.ESHAPE),         # negative group_rows
    ((0, 4, 32, 3, A, None, B, C, D, None, W, WB, None), _abi.ESHAPE),          # 3 does not divide 4
    ((0, 2 ** 40, 2 ** 20, 0, A, None, B, C, D, None, W, WB, None), _abi.ESHAPE),  # N limit
    ((0, 2 ** 20, 2 ** 15 + 16, 0, A, None, B, C, D, None, W, WB, None), _abi.ESHAPE),  # N just above 2^35
    ((0, 4, 32, 0, A, None, B, C, None, None, W, WB, None), _abi.EINVAL),       # NVFP4 needs a gscale
    ((0, 4, 32, 0, A, E, B, C, D, None, W, WB, None), _abi.EINVAL),             # both gscale_in and out
    ((1, 4, 32, 0, A, E, B, C, None, None, None, 0, None), _abi.EINVAL),        # MXFP4 takes no gscale
    ((0, 4, 32, 0, None, None, B, C, D, None, W, WB, None), _abi.EINVAL),       # NULL x
    ((0, 4, 32, 0, A, None, None, C, D, None, W, WB, None), _abi.EINVAL),       # NULL codes
    ((0, 4, 32, 0, A, None, B, C, D, None, None, WB, None), _abi.EINVAL),       # amax needs work
    ((0, 4, 32, 0, A, None, B, C, D, None, W, WB - 4, None), _abi.ESHAPE),      # work too small
    ((0, 6, 32, 3, A, None, B, C, D, None, W, WB, None), _abi.ESHAPE),          # 2 groups need 2*WB
    ((0, 4, 32, 0, A + 8, None, B, C, D, None, W, WB, None), _abi.EALIGN),      # x not 16-B aligned
    ((0, 4, 32, 0, A, None, B + 2, C, D, None, W, WB, None), _abi.EALIGN),      # codes not 4-B aligned
    ((0, 4, 32, 0, A, None, B, C, D, None, W + 4, WB, None), _abi.EALIGN),      # work not 8-B aligned
    ((0, 4, 32, 0, A, None, B, C, D, A + 16, W, WB, None), _abi.EALIAS),        # y overlaps x
    ((0, 4, 32, 0, A, None, B, B + 8, D, None, W, WB, None), _abi.EALIAS),      # scales overlap codes
    ((0, 4, 32, 0, A, None, B, C, A + 4, None, W, WB, None), _abi.EALIAS),      # gscale_out inside x
    ((0, 4, 32, 0, A, None, B, C, D, None, A, WB, None), _abi.EALIAS),          # work over x
    ((0, 4, 32, 0, A, None, B, C, D, None, D - 8, WB, None), _abi.EALIAS),      # work over gscale_out
])
def test_quantize_rtn_rejects(lib, args, status):
    assert lib.quantize_rtn(*args) == status


# encode_guidance(fmt, bits, rows, cols, group_rows, x, gin, guide, scales, gout, y, work, wb, stream)
@pytest.mark.parametrize("args,status", [
    ((0, 5, 4, 32, 0, A, None, B, C, D, None, W, WB, None), _abi.EINVAL),       # bits 5
    ((0, 0, 4, 32, 0, A, None, B, C, D, None, W, WB, None), _abi.EINVAL),       # bits 0
    ((0, 2, 4, 32, 0, A, None, B + 1, C, D, None, W, WB, None), _abi.EALIGN),   # 2-bit plane alignment
    ((0, 3, 4, 32, 0, A, None, B, B + 47, D, None, W, WB, None), _abi.EALIAS),  # 3-bit plane is 48 B
    ((0, 2, 4, 32, 0, A, None, B, B + 31, D, None, W, WB, None), _abi.EALIAS),  # 2-bit plane is 32 B
    ((0, 4, 4, 32, 0, A, None, B + 1, C, D, None, W, WB, None), _abi.EALIGN),   # code plane alignment
    ((0, 1, 4, 32, 0, A, None, B, B + 8, D, None, W, WB, None), _abi.EALIAS),   # bit plane is 16 B here
    ((0, 1, 4, 32, 0, A, None, A + 100, C, D, None, W, WB, None), _abi.EALIAS),
])
def test_encode_guidance_rejects(lib, args, status):
    assert lib.encode_guidance(*args) == status


# decode_guidance(fmt, bits, rows, cols, group_rows, x, guide, scales, gscale, ref, stream)
@pytest.mark.parametrize("args,status", [
    ((0, 1, 4, 32, 0, A, B, C, None, D, None), _abi.EINVAL),            # NVFP4 needs rollout S
    ((1, 1, 4, 32, 0, A, B, C, E, D, None), _abi.EINVAL),               # MXFP4 takes none
    ((0, 0, 4, 32, 0, A, B, C, E, D, None), _abi.EINVAL),               # bits 0 has no record
    ((0, 4, 4, 32, 0, A, B, C, E, D, None), _abi.EINVAL),               # full codes need no decode
    ((0, 1, 4, 32, 0, A, None, C, E, D, None), _abi.EINVAL),            # NULL guide
    ((0, 1, 4, 32, 0, A, B, C, E, None, None), _abi.EINVAL),            # NULL output
    ((0, 1, 4, 32, 3, A, B, C, E, D, None), _abi.ESHAPE),               # grouping
    ((0, 1, 4, 32, 0, A, B, C, E, D + 1, None), _abi.EALIGN),
    ((0, 2, 4, 32, 0, A, B + 1, C, E, D, None), _abi.EALIGN),           # 2-bit plane alignment
    ((0, 1, 4, 32, 0, A, B, C, E, B, None), _abi.EALIAS),               # output on the bits
    ((0, 3, 4, 32, 0, A, B, C, E, B + 44, None), _abi.EALIAS),          # 3-bit plane is 48 B here
])
def test_decode_guidance_rejects(lib, args, status):
    assert lib.decode_guidance(*args) == status


# guided_fake_quant(fmt, bits, rows, cols, group_rows, x, guide, scales, gscale, y, codes, stream)
@pytest.mark.parametrize("args,status", [
    ((0, 5, 4, 32, 0, A, B, C, E, D, None, None), _abi.EINVAL),          # bits 5
    ((0, -1, 4, 32, 0, A, B, C, E, D, None, None), _abi.EINVAL),         # bits -1
    ((0, 0, 4, 32, 0, A, B, C, E, D, None, None), _abi.EINVAL),          # bits 0 takes no guide
    ((0, 3, 4, 32, 0, A, None, C, E, D, None, None), _abi.EINVAL),       # bits 3 needs a guide
    ((0, 2, 4, 32, 0, A, B + 1, C, E, D, None, None), _abi.EALIGN),      # 2-bit guide alignment
    ((0, 3, 4, 32, 0, A, B, C, E, D, B + 40, None), _abi.EALIAS),        # codes over the 3-bit guide
    ((0, 1, 4, 32, 0, A, None, C, E, D, None, None), _abi.EINVAL),       # bits 1 needs a guide
    ((0, 1, 4, 32, 0, A, B, C, E, None, None, None), _abi.EINVAL),       # NULL y
    ((0, 1, 4, 32, 8, A, B, C, E, D, None, None), _abi.ESHAPE),          # 8 does not divide 4
    ((0, 4, 4, 32, 0, A, B + 2, C, E, D, None, None), _abi.EALIGN),      # code guide alignment
    ((0, 1, 4, 32, 0, A, B, C, E, D + 8, None, None), _abi.EALIGN),      # y alignment
    ((0, 1, 4, 32, 0, A, B, C, E, A, None, None), _abi.EALIAS),          # in-place y over x
    ((0, 1, 4, 32, 0, A, B, C, E, D, D + 64, None), _abi.EALIAS),        # codes inside y
    ((0, 1, 4, 32, 0, A, B, C, E, D, C, None), _abi.EALIAS),             # codes over scales
    ((0, 1, 8, 32, 4, A, B, C, E, D, E + 8, None), _abi.EALIAS),         # codes over group 1's S
])
def test_guided_fake_quant_rejects(lib, args, status):
    assert lib.guided_fake_quant(*args) == status


F = 0x700000            # a fake x_rollout address
K = 0x780000            # a fake counts address
SW, SB = W + 4096, 16 * 65 + 4 * 32   # stats workspace address and bytes for [4, 32]
# guided_fake_quant_stats(fmt, bits, rows, cols, group_rows, x, xr, guide, scales, gscale, y, codes,
#                         acc3, counts, accumulate, work, work_bytes, stream)
@pytest.mark.parametrize("args,status", [
    ((0, 1, 4, 32, 0, A, F, B, C, E, D, None, W, None, 2, SW, SB, None), _abi.EINVAL),     # flag
    ((0, 1, 4, 32, 0, A, None, B, C, E, D, None, W, None, 0, SW, SB, None), _abi.EINVAL),  # NULL x_r
    ((0, 1, 4, 32, 0, A, F, B, C, E, D, None, None, K, 0, SW, SB, None), _abi.EINVAL),     # NULL acc
    ((0, 1, 4, 32, 0, A, F, B, C, E, D, None, W, None, 0, None, SB, None), _abi.EINVAL),   # NULL work
    ((0, 1, 4, 32, 0, A, F, B, C, E, D, None, W, None, 0, SW, SB - 8, None), _abi.ESHAPE), # work small
    ((0, 1, 4, 32, 0, A, F + 8, B, C, E, D, None, W, None, 0, SW, SB, None), _abi.EALIGN), # x_r align
    ((0, 1, 4, 32, 0, A, F, B, C, E, D, None, W + 4, None, 0, SW, SB, None), _abi.EALIGN), # acc align
    ((0, 1, 4, 32, 0, A, F, B, C, E, D, None, W, K + 4, 0, SW, SB, None), _abi.EALIGN),    # counts align
    ((0, 1, 4, 32, 0, A, F, B, C, E, F, None, W, None, 0, SW, SB, None), _abi.EALIAS),     # y over x_r
    ((0, 1, 4, 32, 0, A, F, B, C, E, D, None, W, None, 0, W + 8, SB, None), _abi.EALIAS),  # work over acc
    ((0, 1, 4, 32, 0, A, F, B, C, E, D, None, W, W + 16, 0, SW, SB, None), _abi.EALIAS),   # counts over acc
    ((0, 1, 4, 32, 0, A, F, B, C, E, D, None, W, F + 64, 0, SW, SB, None), _abi.EALIAS),   # counts in x_r
    ((0, 1, 4, 32, 0, A, F, B, C, E, D, None, W, SW + 256, 0, SW, SB, None), _abi.EALIAS), # counts in work
])
def test_guided_fake_quant_stats_rejects(lib, args, status):
    assert lib.guided_fake_quant_stats(*args) == status


# discrepancy_stats(n, xt, xr, yt, yr, acc, accumulate, work, work_bytes, stream)
@pytest.mark.parametrize("args,status", [
    ((64, A, B, C, D, E, 2, E + 64, 16, None), _abi.EINVAL),          # accumulate flag
    ((-5, A, B, C, D, E, 0, E + 64, 16, None), _abi.ESHAPE),
    ((64, A, B, C, D, None, 0, E + 64, 16, None), _abi.EINVAL),
    ((64, A, B, C, D, E, 0, None, 16, None), _abi.EINVAL),
    ((64, A, B, C, D, E, 0, E + 64, 8, None), _abi.ESHAPE),           # workspace too small
    ((64, A + 2, B, C, D, E, 0, E + 64, 16, None), _abi.EALIGN),
    ((64, A, B, C, D, E + 4, 0, E + 64, 16, None), _abi.EALIGN),
    ((64, A, B, C, D, A + 8, 0, E + 64, 16, None), _abi.EALIAS),      # acc inside x_t
    ((64, A, B, C, D, E, 0, E + 8, 16, None), _abi.EALIAS),           # work over acc
])
def test_discrepancy_stats_rejects(lib, args, status):
    assert lib.discrepancy_stats(*args) == status


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible: valid calls would launch")
def test_valid_call_without_gpu_is_edevice(lib):
    assert lib.quantize_rtn(0, 4, 32, 0, A, None, B, C, D, None, W, WB, None) == _abi.EDEVICE
    assert lib.encode_guidance(0, 1, 4, 32, 0, A, E, B, C, None, None, None, 0, None) == _abi.EDEVICE
    assert lib.guided_fake_quant(1, 1, 4, 32, 0, A, B, C, None, D, None, None) == _abi.EDEVICE
    assert lib.guided_fake_quant_stats(0, 1, 4, 32, 0, A, F, B, C, E, D, None, W, None, 0, SW, SB,
                                       None) == _abi.EDEVICE
    assert lib.guided_fake_quant_stats(0, 1, 4, 32, 0, A, F, B, C, E, D, None, W, K, 1, SW, SB,
                                       None) == _abi.EDEVICE
    assert lib.decode_guidance(0, 1, 8, 32, 4, A, B, C, E, D, None) == _abi.EDEVICE
    assert lib.discrepancy_stats(64, A, B, C, D, E, 0, E + 64, 16, None) == _abi.EDEVICE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_abi, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _abi.load()


# ---------------------------------------------------------------- record path

def test_ring_rejects_before_any_hip_call(lib):
    h = ctypes.c_void_p(123)
    assert lib.trace_ring_create(1 << 20, 4, None) == _abi.EINVAL
    for sb, n in [(0, 4), (-1, 4), (1, 0), (1, 4097), (1 << 30, 2048)]:
        assert lib.trace_ring_create(sb, n, ctypes.byref(h)) == _abi.ESHAPE, (sb, n)
        assert h.value is None                      # cleared on error
    slot = ctypes.c_int32()
    srcs = (ctypes.c_void_p * 1)(A)
    sizes = (ctypes.c_int64 * 1)(16)
    assert lib.trace_ring_push(None, srcs, sizes, 1, None, ctypes.byref(slot)) == _abi.EINVAL
    assert lib.trace_ring_wait(None, 0) == _abi.EINVAL
    assert lib.trace_ring_query(None, 0) == _abi.EINVAL
    assert lib.trace_ring_release(None, 0) == _abi.EINVAL
    assert lib.trace_ring_slot(None, 0, None) is None
    assert lib.trace_ring_destroy(None) == _abi.EINVAL


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible: a ring would be created")
def test_ring_create_without_gpu_is_edevice(lib):
    h = ctypes.c_void_p()
    assert lib.trace_ring_create(1 << 20, 4, ctypes.byref(h)) == _abi.EDEVICE
    assert h.value is None


# trace_gather_pages(pool, pool_pages, page_bytes, ids, n, out, bad, stream)
@pytest.mark.parametrize("args,status", [
    ((A, 4, 0, B, 2, C, None, None), _abi.ESHAPE),           # page_bytes 0
    ((A, -1, 16, B, 2, C, None, None), _abi.ESHAPE),         # negative pool
    ((A, 4, 16, B, -2, C, None, None), _abi.ESHAPE),         # negative n
    ((A, 4, 1 << 40, B, 1 << 10, C, None, None), _abi.ESHAPE),  # 2^50 bytes
    ((A, 4, 16, None, 2, C, None, None), _abi.EINVAL),       # NULL ids
    ((A, 4, 16, B, 2, None, None, None), _abi.EINVAL),       # NULL out
    ((None, 4, 16, B, 2, C, None, None), _abi.EINVAL),       # NULL pool
    ((A, 4, 16, B + 2, 2, C, None, None), _abi.EALIGN),      # ids alignment
    ((A, 4, 16, B, 2, C, D + 1, None), _abi.EALIGN),         # counter alignment
    ((A, 4, 16, B, 2, A + 48, None, None), _abi.EALIAS),     # out over the pool's last page
    ((A, 4, 16, B, 2, B - 16, None, None), _abi.EALIAS),     # out over the ids
    ((A, 4, 16, B, 2, C, C + 8, None), _abi.EALIAS),         # counter inside out
])
def test_gather_rejects(lib, args, status):
    assert lib.trace_gather_pages(*args) == status


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible: valid calls would launch")
def test_gather_without_gpu_is_edevice(lib):
    assert lib.trace_gather_pages(A, 4, 16, B, 2, C, D, None) == _abi.EDEVICE


# trace_stream_copy(src, dst, bytes, stream) / trace_stream_mix(a, b, out, bytes, stream)
@pytest.mark.parametrize("args,status", [
    ((A, B, 24, None), _abi.ESHAPE),                 # not whole 16-byte words
    ((A, B, -16, None), _abi.ESHAPE),
    ((A, B, (1 << 37) + 16, None), _abi.ESHAPE),     # beyond 2^37 bytes
    ((A, B, 1 << 45, None), _abi.ESHAPE),
    ((None, B, 64, None), _abi.EINVAL),
    ((A, None, 64, None), _abi.EINVAL),
    ((A + 8, B, 64, None), _abi.EALIGN),
    ((A, B + 4, 64, None), _abi.EALIGN),
    ((A, A + 48, 64, None), _abi.EALIAS),            # dst over the source's last word
])
def test_stream_copy_rejects(lib, args, status):
    assert lib.trace_stream_copy(*args) == status


@pytest.mark.parametrize("args,status", [
    ((A, B, C, 40, None), _abi.ESHAPE),
    ((A, None, C, 64, None), _abi.EINVAL),           # the mix needs both sources
    ((None, B, C, 64, None), _abi.EINVAL),
    ((A, B + 8, C, 64, None), _abi.EALIGN),
    ((A, B, B + 16, 64, None), _abi.EALIAS),         # out over the second source
    ((A, A, C, 64, None), _abi.EDEVICE if torch.cuda.device_count() == 0 else _abi.OK),  # one source twice is a read
])
def test_stream_mix_rejects(lib, args, status):
    if status == _abi.OK:
        pytest.skip("a GPU is visible: the call would launch")
    assert lib.trace_stream_mix(*args) == status


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible: valid calls would launch")
def test_stream_references_without_gpu_are_edevice(lib):
    assert lib.trace_stream_copy(A, B, 64, None) == _abi.EDEVICE
    assert lib.trace_stream_mix(A, B, C, 64, None) == _abi.EDEVICE
    assert lib.trace_stream_copy(None, None, 0, None) == _abi.EDEVICE   # even empty: the device is checked


# ---------------------------------------------------------------- row-offset groups

def test_grouped_workspace_sizes(lib):
    # [offs int64 G+1 | tstart int32 G+1 | table int2 x entries | tile maxima u32 x entries],
    # entries = tiles of the call + one per group
    up8 = lambda b: (b + 7) // 8 * 8  # noqa: E731
    for rows, cols, G in [(1000, 2048, 9), (65536, 2048, 256), (4, 32, 1), (64, 32, 4096), (64, 32, 4097)]:
        # [offsets | tile starts | (group, tile) table | tile maxima | S words | flag |
        # descriptors]: the table has the two-pass schedule's entries (TILE-unit tiles);
        # the single pass (up to 4096 groups) adds one 256-byte S line per group, an
        # 8-byte flag and a 16-byte descriptor per 4096-unit tile (on 16 bytes)
        entries = (rows * cols // 8 + TILE - 1) // TILE + G
        single = G <= 4096
        want = up8(8 * (G + 1)) + up8(4 * (G + 1)) + 8 * entries + up8(4 * entries + (256 * G if single else 0))
        if single:
            want = (want + 8 + 15) // 16 * 16 + 16 * ((rows * cols // 8 + 4095) // 4096 + G)
        assert lib.trace_grouped_workspace_bytes(0, rows, cols, G) == want, (rows, cols, G)
    assert lib.trace_grouped_workspace_bytes(1, 64, 2048, 4) == 0
    assert lib.trace_grouped_workspace_bytes(0, 64, 2048, 0) == -1
    assert lib.trace_grouped_workspace_bytes(0, 64, 24, 2) == -1
    # at most 2^22 groups and 2^35 elements per call
    assert lib.trace_grouped_workspace_bytes(0, 2 ** 22, 16, 2 ** 22) > 0
    assert lib.trace_grouped_workspace_bytes(0, 2 ** 22, 16, 2 ** 22 + 1) == -1
    assert lib.trace_grouped_workspace_bytes(0, 2 ** 20, 2 ** 15, 4) > 0
    assert lib.trace_grouped_workspace_bytes(0, 2 ** 20, 2 ** 15 + 16, 4) == -1


def test_size_limits_keep_launches_in_32_bit_grids(lib):
    """2^35 elements is the largest call: its workspaces are defined there and
    not one block beyond (every launch then stays below 2^32 work-items)."""
    assert lib.trace_quant_workspace_bytes(0, 2 ** 20, 2 ** 15, 0) > 0
    assert lib.trace_quant_workspace_bytes(0, 2 ** 20, 2 ** 15 + 16, 0) == -1
    assert lib.trace_guided_stats_workspace_bytes(0, 2 ** 20, 2 ** 15, 0) > 0
    assert lib.trace_guided_stats_workspace_bytes(0, 2 ** 20, 2 ** 15 + 16, 0) == -1
    # 2^35 elements in 1024-unit tiles of 512 threads: 2^22 workgroups, 2^31 work-items
    assert (2 ** 35 // 8 // GTILE) * 512 < 2 ** 32


GW = 0x900000   # fake workspace for the grouped calls
GWB = 1 << 16
O = 0xA00000    # fake device offsets
# encode_guidance_grouped(fmt, bits, rows, cols, G, offs, x, guide, scales, gout, y, work, wb, stream)
@pytest.mark.parametrize("args,status", [
    ((0, 0, 4, 32, 2, O, A, B, C, D, None, GW, GWB, None), _abi.EINVAL),     # bits 0
    ((0, 1, 4, 32, 0, O, A, B, C, D, None, GW, GWB, None), _abi.ESHAPE),    # no groups
    ((0, 1, 4, 32, 2, None, A, B, C, D, None, GW, GWB, None), _abi.EINVAL),  # NULL offsets
    ((0, 1, 4, 32, 2, O, A, B, C, None, None, GW, GWB, None), _abi.EINVAL),  # NVFP4 needs gscale_out
    ((1, 1, 4, 32, 2, O, A, B, C, D, None, None, 0, None), _abi.EINVAL),    # MXFP4 takes none
    ((0, 1, 4, 32, 2, O, A, B, C, D, None, None, GWB, None), _abi.EINVAL),  # NULL work
    ((0, 1, 4, 32, 2, O, A, B, C, D, None, GW, 8, None), _abi.ESHAPE),      # work too small
    ((0, 1, 4, 24, 2, O, A, B, C, D, None, GW, GWB, None), _abi.ESHAPE),    # cols % 16
    ((0, 1, 4, 32, 2, O + 4, A, B, C, D, None, GW, GWB, None), _abi.EALIGN),  # offsets alignment
    ((0, 1, 4, 32, 2, O, A, B, C, D, None, GW + 4, GWB, None), _abi.EALIGN),  # work alignment
    ((0, 1, 4, 32, 2, O, A, B, C, O + 8, None, GW, GWB, None), _abi.EALIAS),  # gscale over offsets
    ((0, 1, 4, 32, 2, O, A, B, C, D, None, A + 64, GWB, None), _abi.EALIAS),  # work over x
])
def test_encode_grouped_rejects(lib, args, status):
    assert lib.encode_guidance_grouped(*args) == status


# guided_fake_quant_grouped(fmt, bits, rows, cols, G, offs, x, guide, scales, gscale, y, codes, work, wb, stream)
@pytest.mark.parametrize("args,status", [
    ((0, 5, 4, 32, 2, O, A, B, C, E, D, None, GW, GWB, None), _abi.EINVAL),    # bits 5
    ((0, 1, 4, 32, -1, O, A, B, C, E, D, None, GW, GWB, None), _abi.ESHAPE),  # negative groups
    ((0, 1, 4, 32, 2, None, A, B, C, E, D, None, GW, GWB, None), _abi.EINVAL),  # NULL offsets
    ((0, 1, 4, 32, 2, O, A, B, C, None, D, None, GW, GWB, None), _abi.EINVAL),  # NVFP4 needs gscale
    ((0, 0, 4, 32, 2, O, A, B, C, E, D, None, GW, GWB, None), _abi.EINVAL),    # bits 0 takes no guide
    ((0, 1, 4, 32, 2, O, A, B, C, E, None, None, GW, GWB, None), _abi.EINVAL),  # NULL y
    ((0, 1, 4, 32, 2, O, A, B, C, E, D, None, GW, 8, None), _abi.ESHAPE),      # work too small
    ((0, 1, 4, 32, 2, O, A, B, C, E, D + 8, None, GW, GWB, None), _abi.EALIGN),  # y alignment
    ((0, 1, 4, 32, 2, O, A, B, C, E, O, None, GW, GWB, None), _abi.EALIAS),    # y over offsets
    ((0, 1, 4, 32, 2, O, A, B, C, E, D, None, E, GWB, None), _abi.EALIAS),     # work over gscale
])
def test_guided_grouped_rejects(lib, args, status):
    assert lib.guided_fake_quant_grouped(*args) == status


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is visible: valid calls would launch")
def test_grouped_without_gpu_is_edevice(lib):
    assert lib.encode_guidance_grouped(0, 1, 4, 32, 2, O, A, B, C, D, None, GW, GWB, None) == _abi.EDEVICE
    assert lib.guided_fake_quant_grouped(0, 1, 4, 32, 2, O, A, B, C, E, D, None, GW, GWB, None) == _abi.EDEVICE
