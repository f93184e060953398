"""Host-side checks of bench.py: the one-GPU guard and the counter summaries it reads.

No GPU is used: the guard exits before any device call, and the traffic
figures come from text files next to the kernel source's digest.
"""

import hashlib
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _fake_tree(tmp_path, source: bytes, summary: str):
    (tmp_path / "invariant_gemm_token_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "invariant_gemm_token_amd" / "csrc" / "tig_kernels.hip").write_bytes(source)
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "demo_traffic.md").write_text(summary)


def test_traffic_is_read_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch):
    bench = _bench()
    src = b"// kernel source\n"
    digest = hashlib.sha256(src).hexdigest()
    _fake_tree(tmp_path, src, f"# demo\n\ntraffic_bytes_per_launch: 1.5e+09\nkernel_source_sha256: `{digest}`\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("demo") == 1.5e9
    # the source changed since the counters were taken: no figure
    (tmp_path / "invariant_gemm_token_amd" / "csrc" / "tig_kernels.hip").write_bytes(src + b"// edit\n")
    assert bench.measured_traffic("demo") is None
    # no summary at all
    assert bench.measured_traffic("absent") is None


def test_unparsable_traffic_gives_none(tmp_path, monkeypatch):
    bench = _bench()
    src = b"x"
    digest = hashlib.sha256(src).hexdigest()
    _fake_tree(tmp_path, src, f"traffic_bytes_per_launch: n/a\nkernel_source_sha256: `{digest}`\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("demo") is None


@pytest.mark.parametrize("name", ["lmhead_prefill", "lmhead_decode", "tree_gemm_lmhead"])
def test_committed_summaries_carry_both_fields(name):
    text = open(os.path.join(ROOT, "profiles", f"{name}_traffic.md")).read()
    fields = {}
    for line in text.splitlines():
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    assert float(fields["traffic_bytes_per_launch"]) > 0
    assert len(fields["kernel_source_sha256"]) == 64
    assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text
