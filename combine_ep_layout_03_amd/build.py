"""Build the HIP library in-tree: combine_ep_layout_03_amd/libep_mi355x.so.

One hipcc invocation for gfx950 only.  Floating-point flags matter for
bit-exact results: no contraction of a*b+c into FMA, correctly rounded fp32
division, fp32 denormals kept, no fast-math, and no packed-fp32 instructions.
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libep_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["ep_api.hip", "ep_layout.hip", "ep_dispatch.hip", "ep_combine.hip", "ep_gemm.hip"]

# test-only library exposing the device E4M3FN encoders (tests/hip)
TEST_SOURCE = os.path.join(ROOT, "tests", "hip", "e4m3_check.hip")
TEST_LIB_PATH = os.path.join(ROOT, "tests", "hip", "libep_e4m3_check.so")

# plain-C consumer of the C ABI (tests/c), built with the host C compiler
C_EXAMPLE_SOURCE = os.path.join(ROOT, "tests", "c", "ep_c_roundtrip.c")
C_EXAMPLE_PATH = os.path.join(ROOT, "tests", "c", "ep_c_roundtrip")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
# what a C (not HIP) translation unit needs to include the HIP runtime API
C_HIP_FLAGS = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str | None = None) -> str:
    """Compile every source into the shared library and return its path."""
    out = out or LIB_PATH
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", INCLUDE, "-I", CSRC]
    cmd += [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    if verbose and (res.stdout or res.stderr):
        print(res.stdout, res.stderr, flush=True)
    os.replace(tmp, out)
    return out


def build_test_lib(verbose: bool = False) -> str:
    """Compile the test-only encoder library with the product's flags."""
    tmp = TEST_LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, TEST_SOURCE, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, TEST_LIB_PATH)
    return TEST_LIB_PATH


def build_c_example(verbose: bool = False) -> str:
    """Compile the C99 program that drives the library through the header
    alone (layout, dispatch, combine); links the in-tree library by rpath."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler found for the C-ABI example")
    tmp = C_EXAMPLE_PATH + ".tmp"
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Wextra", *C_HIP_FLAGS, "-I", INCLUDE, C_EXAMPLE_SOURCE,
           "-o", tmp, "-L", HERE, "-lep_mi355x", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../combine_ep_layout_03_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C build failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, C_EXAMPLE_PATH)
    return C_EXAMPLE_PATH


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_test_lib(verbose=True))
    print(build_c_example(verbose=True))
