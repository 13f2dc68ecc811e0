"""Build libtrace_fp4.so in-tree with hipcc for gfx950.

    python -m precision_rl_nvfp4_amd.build

Flags that matter for bit-exact results:
  -ffp-contract=off   no fused multiply-add: every binary32 operation rounds
                      on its own, as the ABI documents
  (default)           fp32 denormals are kept and fp32 division is correctly
                      rounded (hipcc's defaults; no fast-math flags are given)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed FP32 instructions (v_pk_add/mul/fma_f32) in
                      device code; hipcc -O3 forms them from plain float
                      code otherwise. The host passes do not know the feature
                      and say so ("not a recognized feature"); the device pass
                      honours it. build() checks the result: it keeps the
                      device assembly of the build and fails if any of the
                      three instructions appears in it.
"""

from __future__ import annotations

import glob
import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtrace_fp4.so")
SOURCES = [os.path.join(CSRC, "trace_fp4_kernels.hip"), os.path.join(CSRC, "trace_fp4_api.cpp"),
           os.path.join(CSRC, "trace_fp4_record.hip"), os.path.join(CSRC, "trace_fp4_stream.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def command(out: str = LIB, extra=()) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", *NO_PACKED_FP32, "-Wall", "-Wno-unused-function", *extra,
            "-I", os.path.join(ROOT, "include"), "-o", out] + SOURCES


def packed_fp32_lines(asm_dir: str) -> list[str]:
    """Lines of the device assembly files in asm_dir that hold a packed FP32
    instruction."""
    hits = []
    for path in sorted(glob.glob(os.path.join(asm_dir, f"*-hip-amdgcn-amd-amdhsa-{ARCH}.s"))):
        with open(path) as f:
            hits += [f"{os.path.basename(path)}: {l.strip()}" for l in f if PACKED_FP32.search(l)]
    return hits


def build(verbose: bool = False) -> str:
    """Compile the library (always, even if a built copy exists), check that
    its device code holds no packed FP32 instruction, and return its path."""
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="trace_fp4_build_") as work:
        cmd = command(tmp, ("-save-temps",))
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True, cwd=work)
        # the host passes' note on the device-only feature (see the docstring)
        noise = "'-packed-fp32-ops' is not a recognized feature"
        errs = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
        asm = glob.glob(os.path.join(work, f"*-hip-amdgcn-amd-amdhsa-{ARCH}.s"))
        if len(asm) != len(SOURCES):
            raise RuntimeError(f"expected the device assembly of {len(SOURCES)} sources, found {len(asm)}")
        hits = packed_fp32_lines(work)
        if hits:
            os.unlink(tmp)
            raise RuntimeError("packed FP32 instructions in device code:\n" + "\n".join(hits[:20]))
    os.replace(tmp, LIB)
    return LIB


# Host-side sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer on
# the host code only; device code is compiled as usual). It is loaded by the
# CPU tests of the C ABI's argument checking, never on a GPU.
SAN_LIB = os.path.join(PKG, "_build", "libtrace_fp4_hostsan.so")
SAN_FLAGS = ("-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer", "-g")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime a host process must preload to load
    the sanitizer build."""
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "llvm")
    cands = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not cands:
        cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return cands[-1]


def build_sanitized(verbose: bool = False) -> str:
    """Compile the host-sanitizer variant of the library into SAN_LIB."""
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    tmp = SAN_LIB + ".tmp"
    cmd = command(tmp, SAN_FLAGS)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc (host sanitizers) failed ({res.returncode}):\n{res.stderr[-4000:]}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--host-sanitizers":
        print(build_sanitized(verbose=True))
    else:
        print(build(verbose=True))
