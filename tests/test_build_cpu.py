"""The build flags, checked with the compiler itself (hipcc cross-compiles
gfx950 without a GPU): the device pass honours the flag that disables packed
FP32 instructions (a float2 multiply-add compiles to v_pk_fma_f32 without it
and to none with it), and the library's own device assembly holds none."""

import os
import subprocess

import pytest

from precision_rl_nvfp4_amd import build as B

KERNEL = """
#include <hip/hip_runtime.h>
__global__ void k(float2* a, const float2* b, const float2* c) {
  const int i = threadIdx.x + blockIdx.x * blockDim.x;
  const float2 x = b[i], y = c[i];
  a[i] = make_float2(x.x * y.x + 1.0f, x.y * y.y + 1.0f);
}
"""


def _device_asm(tmp_path, flags):
    src = tmp_path / "k.hip"
    src.write_text(KERNEL)
    out = tmp_path / f"k{len(flags)}.s"
    subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-O3", "-ffp-contract=fast", "--cuda-device-only",
                    "-S", "-o", str(out), str(src), *flags], check=True, capture_output=True, text=True)
    return out.read_text()


@pytest.fixture(scope="module")
def have_hipcc():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")


def test_flag_removes_packed_fp32_from_device_code(have_hipcc, tmp_path):
    without = _device_asm(tmp_path, [])
    with_flag = _device_asm(tmp_path, B.NO_PACKED_FP32)
    assert B.PACKED_FP32.search(without), "the probe kernel should use a packed FP32 op by default"
    assert not B.PACKED_FP32.search(with_flag)


def test_library_build_command_carries_the_flag():
    cmd = B.command("/dev/null")
    i = cmd.index("-target-feature")
    assert cmd[i - 1:i + 3] == B.NO_PACKED_FP32
    assert "-ffp-contract=off" in cmd


def test_library_device_assembly_has_no_packed_fp32(have_hipcc, tmp_path):
    """The library's kernel source through the same device pass as build()."""
    src = os.path.join(B.CSRC, "trace_fp4_kernels.hip")
    out = tmp_path / f"trace_fp4_kernels-hip-amdgcn-amd-amdhsa-{B.ARCH}.s"
    subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-O3", "-std=c++17", "-ffp-contract=off",
                    *B.NO_PACKED_FP32, "--cuda-device-only", "-S", "-I", os.path.join(B.ROOT, "include"),
                    "-o", str(out), src], check=True, capture_output=True, text=True)
    assert B.packed_fp32_lines(str(tmp_path)) == []
