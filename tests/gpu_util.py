"""Helpers for the GPU tests: device transfer, bitwise comparison, diff metrics.

Bitwise comparison follows the bit-consistent RL post, section 2: the per-token
difference must be exactly zero (max, mean and std of |delta| and the k3 KL),
which is checked on the raw bits; on failure the first differing index and
value pair are reported.
"""

import os
import sys

import numpy as np
import torch


# Every comparison made through these helpers during a test session, written
# as JSON at the end of the session (tests/conftest.py): the bitwise checks
# with their diff statistics (max, mean, std of |delta| and the k3 KL of the
# bit-consistent RL post, section 3.2, all exactly 0 when they pass) and the
# largest deviations from the fp64 oracle.
REPORT: list = []


def record(kind: str, what: str, **fields):
    """Add one comparison to the session report, tagged with the running test."""
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    REPORT.append(dict(test=test, kind=kind, what=what, **fields))


def say(*a):
    """Print and flush, so that the case being run is visible even if the run dies."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> bfloat16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a float32 / bf16 / int32 tensor as an unsigned numpy array."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)


def assert_bitwise(a: torch.Tensor, b: torch.Tensor, what: str):
    ba, bb = host_bits(a), host_bits(b)
    assert ba.shape == bb.shape, f"{what}: shapes {ba.shape} vs {bb.shape}"
    fields = {"elements": int(ba.size), "differing": int(np.count_nonzero(ba != bb))}
    if a.dtype == torch.float32 and a.dim() == 1:
        fields.update(diff_stats(a.detach().cpu().double().numpy(), b.detach().cpu().double().numpy()))
    record("bitwise", what, **fields)
    if not np.array_equal(ba, bb):
        idx = np.argwhere(ba != bb)
        i = tuple(idx[0])
        va = a.detach().cpu()[i].item()
        vb = b.detach().cpu()[i].item()
        raise AssertionError(f"{what}: {len(idx)} elements differ; first at {i}: {va!r} vs {vb!r}")


def diff_stats(a, b) -> dict:
    """max / mean / std of |a - b| and the mean k3 KL between logprob vectors."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    d = np.abs(a - b)
    r = b - a
    return {"max": float(d.max()) if d.size else 0.0, "mean": float(d.mean()) if d.size else 0.0,
            "std": float(d.std()) if d.size else 0.0,
            "k3": float(np.mean(np.expm1(r) - r)) if d.size else 0.0}


def assert_gemm_close(got: np.ndarray, ref: np.ndarray, rel: float = 2e-3, what: str = "gemm"):
    """Elementwise |got - ref| <= rel * max(|ref|, rms(ref)) (the GEMM parity bar)."""
    got = np.asarray(got, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = rel * np.maximum(np.abs(ref), rms)
    bad = np.abs(got - ref) > bound
    worst = float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), rms))) if ref.size else 0.0
    record("oracle_gemm", what, elements=int(ref.size), max_rel=worst, bound=rel, outside=int(bad.sum()))
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} outside tolerance; first {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} bound {bound[i]!r}")
    return worst
