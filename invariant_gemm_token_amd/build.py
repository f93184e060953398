"""Build libtig.so in-tree: hand-written HIP kernels for gfx950 plus the host-side C ABI.

``python -m invariant_gemm_token_amd.build`` compiles every source each time it
is called.  The device code is compiled with packed-FP32 instructions disabled
and floating-point contraction off; the host part is plain C++17.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtig.so")
# A C99 client of the ABI (tests/c_abi), linked against the library: the GPU
# tests run it as a program of its own.
CLIENT_SRC = os.path.join(ROOT, "tests", "c_abi", "tig_c_client.c")
CLIENT = os.path.join(ROOT, "tests", "c_abi", "tig_c_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core accumulators in VGPRs: the leaf-tree adds then need no
    # AGPR<->VGPR copies, which frees ~80 registers per lane.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-Wall",
              f"-I{ROCM}/include"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose and (r.stdout.strip() or r.stderr.strip()):
        print(r.stdout + r.stderr, flush=True)


def build(verbose: bool = False) -> str:
    """Compile the kernels and the C ABI into ``invariant_gemm_token_amd/libtig.so``, and
    the C client of the ABI into ``tests/c_abi/tig_c_client``."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = [f"-I{INCLUDE}", f"-I{CSRC}"]
    kobj = os.path.join(BUILD_DIR, "tig_kernels.o")
    hobj = os.path.join(BUILD_DIR, "tig_api.o")
    _run([HIPCC, "-c", os.path.join(CSRC, "tig_kernels.hip"), "-o", kobj] + DEVICE_FLAGS + inc, verbose)
    _run(["g++", "-c", os.path.join(CSRC, "tig_api.cpp"), "-o", hobj] + HOST_FLAGS + inc, verbose)
    tmp = LIB + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, kobj, hobj,
          f"-L{ROCM}/lib", "-lamdhip64", "-Wl,--no-undefined"], verbose)
    shutil.move(tmp, LIB)
    if os.path.exists(CLIENT_SRC):
        ctmp = CLIENT + ".tmp"
        _run(["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
              f"-I{ROCM}/include", CLIENT_SRC, "-o", ctmp, f"-L{PKG}", "-ltig", f"-L{ROCM}/lib", "-lamdhip64",
              "-lm", "-Wl,-rpath,$ORIGIN/../../invariant_gemm_token_amd", f"-Wl,-rpath,{ROCM}/lib"], verbose)
        shutil.move(ctmp, CLIENT)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
