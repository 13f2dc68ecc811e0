"""Build libtrace_fp4.so in-tree with hipcc for gfx950.

    python -m precision_rl_nvfp4_amd.build

Flags that matter for bit-exact results:
  -ffp-contract=off   no fused multiply-add: every binary32 operation rounds
                      on its own, as the ABI documents
  (default)           fp32 denormals are kept and fp32 division is correctly
                      rounded (hipcc's defaults; no fast-math flags are given)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed FP32 instructions in device code
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtrace_fp4.so")
SOURCES = [os.path.join(CSRC, "trace_fp4_kernels.hip"), os.path.join(CSRC, "trace_fp4_api.cpp"),
           os.path.join(CSRC, "trace_fp4_record.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def command(out: str = LIB) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), "-o", out] + SOURCES


def build(verbose: bool = False) -> str:
    """Compile the library (always, even if a built copy exists) and return its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    errs = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
