"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tig_api.cpp (argument validation, the policy descriptor and its SHA-256,
workspace queries, error strings) is compiled with g++ and
-fsanitize=address,undefined into a CPU-only library whose kernel launchers
are stubs (tests/sanitize/host_stubs.cpp), and the host ABI tests
(tests/test_abi_host.py) run against it in a child process with the sanitizer
runtime preloaded.  Any out-of-bounds access, use of freed memory, overflow
or other undefined behaviour reached by those tests aborts the child.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "invariant_gemm_token_amd", "csrc")


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_abi_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("g++ sanitizer runtimes not installed")
    lib = str(tmp_path / "libtig_host_sanitized.so")
    cmd = ["g++", "-shared", "-fPIC", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "tig_api.cpp"), os.path.join(ROOT, "tests", "sanitize", "host_stubs.cpp"),
           "-o", lib]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr
    env = dict(os.environ)
    env.update({
        "TIG_LIB": lib,
        "LD_PRELOAD": f"{asan}:{ubsan}",
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "HIP_VISIBLE_DEVICES": "",
        "TIG_TEST_REPORT": str(tmp_path / "report.json"),
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_host.py"),
                        "-q", "-p", "no:cacheprovider", "-x"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
