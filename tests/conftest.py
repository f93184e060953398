import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (seconds to minutes)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on cuda:0; a GPU test fails loudly if either is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no GPU is visible")
    import invariant_gemm_token_amd as tig
    tig.load()  # raises if libtig.so is missing or does not load
    return tig


def pytest_sessionfinish(session, exitstatus):
    """Write the session's comparison report (bitwise diff statistics and oracle
    deviations) as JSON: $TIG_TEST_REPORT, else gpurun_out/gpu_test_report.json."""
    gu = sys.modules.get("gpu_util")
    if gu is None or not getattr(gu, "REPORT", None):
        return
    import json
    recs = gu.REPORT
    bit = [r for r in recs if r["kind"] == "bitwise"]
    summary = {
        "bitwise_checks": len(bit),
        "bitwise_elements": sum(r["elements"] for r in bit),
        "bitwise_differing": sum(r["differing"] for r in bit),
        "max_abs_diff": max((r.get("max", 0.0) for r in bit), default=0.0),
        "max_k3": max((abs(r.get("k3", 0.0)) for r in bit), default=0.0),
        "oracle_max_abs_logprob": max((r["max_abs_logprob"] for r in recs if r["kind"] == "oracle_logprob"),
                                      default=None),
        "oracle_max_rel_gemm": max((r["max_rel"] for r in recs if r["kind"] == "oracle_gemm"), default=None),
    }
    out = {"exitstatus": int(exitstatus), "host_cores": os.cpu_count(), "summary": summary, "records": recs}
    try:
        import torch
        if torch.cuda.is_available():
            out["device"] = torch.cuda.get_device_name(0)
    except Exception:
        pass
    path = os.environ.get("TIG_TEST_REPORT") or os.path.join(ROOT, "gpurun_out", "gpu_test_report.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
