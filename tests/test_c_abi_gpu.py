"""GPU: the C client of the ABI (tests/c_abi/tig_c_client.c, built by
__graft_entry__.build()) runs tig_tree_gemm and tig_logprob_gather from C, in a
process of its own, and checks them against values fixed by arithmetic: exact
integer contractions at 1, 8 and 16 leaves, and logprob -ln V when every logit
is equal ([BitRL, section 2])."""

import os
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_abi", "tig_c_client")


def test_c_client_runs_the_gpu_path():
    if not os.path.exists(CLIENT):
        pytest.fail("tests/c_abi/tig_c_client is not built: run __graft_entry__.build()")
    say("C client --gpu")
    r = subprocess.run([CLIENT, "--gpu"], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert "gpu: tree GEMM exact" in r.stdout and r.stdout.strip().endswith("ok")
