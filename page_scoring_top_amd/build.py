"""Build libpagescore.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python page_scoring_top_amd/build.py

(run by path: importing the package loads the library, which may not exist
yet or may predate a new entry point)

Every source under csrc/ is compiled by hipcc to an object, in parallel, and
the objects are linked into page_scoring_top_amd/libpagescore.so.  Packed FP32
instructions are disabled for device code (-packed-fp32-ops).
"""

from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpagescore.so")
BUILD_DIR = os.path.join(PKG, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpagescore.so")


def common_flags():
    # MFMA results in VGPRs: the epilogues read every accumulator, and the
    # AGPR form would add one v_accvgpr_read per value.
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-I", INCLUDE, "-I", CSRC]


# Extra flags for single sources (none at present).
FILE_FLAGS: dict = {}


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        cmd = [cc, *common_flags(), *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose:
            print(" ".join(cmd))
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def build_test_probe() -> str:
    """tests/probe/libmfma_probe.so: the test suite's matrix-instruction
    accuracy probe (not part of the library)."""
    src = os.path.join(ROOT, "tests", "probe", "mfma_accuracy.hip")
    out = os.path.join(ROOT, "tests", "probe", "libmfma_probe.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
