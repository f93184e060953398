"""The C ABI from C: include/tig.h compiles as C99 with every warning on, and a
C program linked against libtig.so runs the host-side calls (workspace
queries, argument errors, the plan descriptor) with no GPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
PKG = os.path.join(ROOT, "invariant_gemm_token_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_is_c99_and_host_calls_work_from_c(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libtig.so")):
        pytest.fail("libtig.so is not built: run __graft_entry__.build()")
    exe = str(tmp_path / "tig_c_client")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-pedantic", "-Wno-long-long",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", "-isystem", f"{ROCM}/include",
           os.path.join(ROOT, "tests", "c_abi", "tig_c_client.c"), "-o", exe, f"-L{PKG}", "-ltig",
           f"-L{ROCM}/lib", "-lamdhip64", "-lm", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ROCM}/lib"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
