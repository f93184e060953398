"""GPU parity and batch invariance of tig_topk_positions (deterministic Top-K).

[BitRL, section 4.3]: the sparse-attention indexer keeps at most 2048
positions per query; the selection key is the score together with the
in-request position, so equal scores go to the larger position, and the
selected positions are listed by descending position with invalid entries
last.  The result is integer: every case must match the oracle exactly.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(gpu_lib, scores: np.ndarray, lengths: np.ndarray, k: int) -> np.ndarray:
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).to(DEV)
    n = torch.from_numpy(np.ascontiguousarray(lengths, dtype=np.int32)).to(DEV)
    out = gpu_lib.topk_positions(s, n, k)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.int64)


def _check(gpu_lib, scores, lengths, k, what):
    say(f"topk {what}: R={scores.shape[0]} ld={scores.shape[1]} k={k}")
    got = _run(gpu_lib, scores, lengths, k)
    ref = oracle.topk_positions(scores, lengths, k)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, (what, bad[:4].tolist(), got[tuple(bad[0])], ref[tuple(bad[0])])
    return got


@pytest.mark.parametrize("grid,ld,k", [
    ("bf16", 1000, 7),        # one partial group of slots
    ("int", 8193, 2048),      # ties everywhere, one position past a full group
    ("bf16", 513, 2048),      # k above every length: all positions, then -1
    ("int", 65536, 1),        # k = 1 over the longest rows
    ("bf16", 4096, 4096),     # k equal to the row length
    ("f32", 20000, 2048),     # (almost) no ties
    ("int", 2048, 2047),
])
def test_topk_matches_oracle(gpu_lib, grid, ld, k):
    rng = np.random.default_rng(7000 + ld + k)
    R = 24
    scores = wl.indexer_scores(rng, R, ld, grid)
    edges = [0, 1, 2, k - 1, k, k + 1, ld - 1, ld, 511, 512, 513, 8191, 8192, 8193]
    lengths = np.array([e for e in edges if 0 <= e <= ld] + list(rng.integers(0, ld + 1, size=R)),
                       dtype=np.int32)[:R]
    _check(gpu_lib, scores, lengths, k, f"{grid}")


def test_topk_special_values(gpu_lib):
    """NaN after every number, +0 equal to -0, infinities and the extremes in place."""
    rng = np.random.default_rng(7100)
    R, ld, k = 16, 3000, 64
    scores = wl.indexer_scores(rng, R, ld, "int")
    specials = np.array([np.nan, 0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max,
                         -np.finfo(np.float32).max, np.finfo(np.float32).tiny, 1e-45, -1e-45], dtype=np.float32)
    for r in range(R):
        idx = rng.choice(ld, size=ld // (r + 2), replace=False)
        scores[r, idx] = rng.choice(specials, size=idx.size)
    scores[0] = np.nan                              # only NaN: every position ties
    scores[1] = -0.0
    scores[1, ::3] = 0.0                            # +0 and -0 tie
    scores[2, :] = -np.inf
    scores[2, 100:110] = np.nan                     # NaN below -inf
    lengths = np.full(R, ld, dtype=np.int32)
    lengths[3] = 40                                 # fewer than k
    got = _check(gpu_lib, scores, lengths, k, "special values")
    assert np.array_equal(got[0], np.arange(ld - 1, ld - 1 - k, -1))
    assert got[2, -1] == ld - 1 - (k - 1) and 100 not in got[2]


def test_topk_lengths_clamped(gpu_lib):
    """Lengths below 0 count as 0 (all -1), above the row pitch as the pitch."""
    rng = np.random.default_rng(7200)
    ld, k = 700, 16
    scores = wl.indexer_scores(rng, 4, ld)
    lengths = np.array([-5, 0, ld + 9, 2 ** 31 - 1], dtype=np.int32)
    got = _run(gpu_lib, scores, lengths, k)
    assert np.all(got[:2] == -1)
    clamp = np.clip(lengths, 0, ld)
    assert np.array_equal(got, oracle.topk_positions(scores, clamp, k))


def test_topk_row_position_invariance(gpu_lib):
    """A request's result depends on its own scores only: not on its row in the
    batch, its neighbours, the batch size, the row pitch or what lies past its
    length."""
    rng = np.random.default_rng(7300)
    k = 2048
    reqs = [wl.indexer_scores(rng, 1, n, g)[0] for n, g in
            ((5000, "bf16"), (65536, "int"), (1234, "bf16"), (30000, "f32"), (2048, "int"))]
    alone = [_run(gpu_lib, q[None, :], np.array([q.size], np.int32), k)[0] for q in reqs]
    ld = 65536
    for trial in range(3):
        R = 9 + 4 * trial
        batch = wl.indexer_scores(rng, R, ld, "bf16")   # other requests around them
        lengths = wl.request_lengths(rng, R, 0, ld)
        slots = rng.choice(R, size=len(reqs), replace=False)
        for q, sl in zip(reqs, slots):
            batch[sl, :q.size] = q
            batch[sl, q.size:] = rng.standard_normal(ld - q.size)   # garbage past the length
            lengths[sl] = q.size
        say(f"topk invariance trial {trial}: R={R} ld={ld}")
        got = _run(gpu_lib, batch, lengths, k)
        for q, sl, a in zip(reqs, slots, alone):
            assert np.array_equal(got[sl], a), (trial, q.size, int(sl))
        assert np.array_equal(got, oracle.topk_positions(batch, lengths, k))


def test_topk_repeat_calls_identical(gpu_lib):
    rng = np.random.default_rng(7400)
    scores = wl.indexer_scores(rng, 64, 65536, "int")
    lengths = wl.request_lengths(rng, 64, 0, 65536)
    first = _run(gpu_lib, scores, lengths, 2048)
    for _ in range(3):
        assert np.array_equal(_run(gpu_lib, scores, lengths, 2048), first)


@pytest.mark.slow
def test_topk_indexer_config(gpu_lib):
    """The indexer workload the bench times (128 rows, pitch 65536, k = 2048,
    lengths mixed), every row against the oracle."""
    c = wl.CONFIGS["indexer"]
    s = wl.streams(c.seed)
    scores = wl.indexer_scores(s["scores"], c.tokens, c.N)
    lengths = wl.request_lengths(s["lengths"], c.tokens, 1, c.N)
    lengths[:4] = (c.N, c.topk, c.topk - 1, 1)
    _check(gpu_lib, scores, lengths, c.topk, "indexer config")


def test_topk_threshold_bin_beyond_the_list(gpu_lib):
    """Rows whose threshold lies in one first-pass key bin holding more keys than
    the LDS list of the last two passes takes (14364): they scan every key again.
    Floats in [1, 1 + 2^-4) share sign, exponent and the top four mantissa
    bits, so every key of such a row falls in one bin of the first digit (the
    key's top 11 bits); lengths straddle the list's size, and reach past it by
    10000 and more."""
    rng = np.random.default_rng(7200)
    R, ld, k = 10, 65536, 2048
    mant = rng.integers(0, 1 << 19, size=(R, ld)).astype(np.uint32)
    scores = (np.uint32(0x3F800000) | mant).view(np.float32)
    scores[1] = 1.0                                  # one key everywhere: ties by position
    scores[2, ::2] = 2.0                             # half the row in a higher bin, all equal
    lengths = np.array([ld, ld, ld, 20000, 14365, 14364, 24589, 24588, 30000, 65535], dtype=np.int32)
    _check(gpu_lib, scores, lengths, k, "one dense bin")


# The kernel first bounds T from below with a sample of each row (slot 4w of
# every thread of wave w: positions n-1-(4160w + l), l < 64) and, when at most
# 8192 keys reach that bound, runs its radix passes over those keys alone.
# The mirror below follows that rule on the host, only to make sure that each
# case here takes the path it is meant to take; the expected result comes from
# the oracle alone.
def _sampled_positions(n: int) -> np.ndarray:
    p = np.array([n - 1 - (4160 * w + l) for w in range(16) for l in range(64)])
    return p[p >= 0]


def _takes_list_path(row: np.ndarray, n: int, k: int) -> bool:
    take = min(n, k)
    m = _sampled_positions(n).size
    rs = 3 * take * m // (2 * n) + 8
    if m < 256 or 4 * rs > m:
        return False
    x = row[:n].astype(np.float32)
    b = (x + np.float32(0)).view(np.uint32)
    key = b ^ (((b.view(np.int32) >> 31).view(np.uint32)) | np.uint32(0x80000000))
    key = np.where(np.isnan(x), np.uint32(1), key).astype(np.uint32)
    ds = int(np.sort(key[_sampled_positions(n)] >> 21)[::-1][rs - 1])
    if ds == 0:
        return False
    total = int((key >= np.uint32(ds << 21)).sum())
    return take <= total <= 8192


def test_topk_sampled_bound_both_paths(gpu_lib):
    """Rows built so that the sample's bound is right, too high (fewer than k
    keys reach it), too low (more keys than the list holds), and at the list's
    capacity exactly (all ties at T) and one past it, plus list-path rows with
    T among denormals and zeros, below zero, and at -inf among NaN: every row
    must match the oracle whichever path it takes."""
    rng = np.random.default_rng(7500)
    ld, k = 65536, 2048
    sp = _sampled_positions(ld)
    rows, want = [], []
    rows.append(rng.standard_normal(ld).astype(np.float32)); want.append(True)        # plain N(0, 1)
    r = rng.standard_normal(ld).astype(np.float32); r[sp] = 50.0 + rng.random(sp.size, dtype=np.float32)
    rows.append(r); want.append(False)                                              # bound too high
    r = rng.standard_normal(ld).astype(np.float32); r[sp] = -50.0
    rows.append(r); want.append(False)                                              # bound too low
    for extra, w in ((8192 - sp.size, True), (8193 - sp.size, False)):              # at / past capacity
        r = np.full(ld, -1.0, np.float32)
        others = np.setdiff1d(np.arange(ld), sp)
        r[sp] = 1.0
        r[rng.choice(others, size=extra, replace=False)] = 1.0
        rows.append(r); want.append(w)
    r = rng.standard_normal(ld).astype(np.float32); r[::7] = np.nan                 # NaN among the keys
    rows.append(r); want.append(True)
    # The list path compares score bits as floats against the bound and T:
    # T among denormals and signed zeros, ...
    r = np.full(ld, -1.0, np.float32)
    tiny = np.array([1, 2, 3, 100, 0x1000, 0x1FFFFF], np.uint32).view(np.float32)   # one first-digit bin
    at = np.union1d(sp, rng.choice(ld, size=3000, replace=False))
    r[at] = rng.choice(np.concatenate([tiny, np.float32([0.0, -0.0])]), size=at.size)
    big = np.array([0x400000, 0x7FFFFF], np.uint32).view(np.float32)                 # larger denormals
    r[rng.choice(np.setdiff1d(np.arange(ld), sp), size=40, replace=False)] = rng.choice(big, size=40)
    rows.append(r); want.append(True)
    r = -np.exp(rng.standard_normal(ld)).astype(np.float32)                       # ... every score negative, ...
    rows.append(r); want.append(True)
    r = np.full(ld, np.nan, np.float32)                                             # ... and T = -inf among NaN
    at = np.union1d(sp, rng.choice(ld, size=4500, replace=False))
    r[at] = -np.inf
    r[rng.choice(np.setdiff1d(np.arange(ld), sp), size=1000, replace=False)] = rng.standard_normal(1000)
    rows.append(r); want.append(True)
    # bf16-valued scores (every key ends in 16 zero bits, so the last pass can
    # be skipped) with float32 values, whose low bits are set, well above the
    # threshold (the skip still holds) or inside the threshold's first-digit
    # bin, [1.75, 2) here (the last pass must run).
    base = wl.indexer_scores(rng, 2, ld, "bf16")
    r = base[0].copy()
    r[rng.choice(ld, size=50, replace=False)] = np.float32(10.0) + rng.random(50, dtype=np.float32) * np.float32(1e-3)
    rows.append(r); want.append(True)
    r = base[1].copy()
    r[rng.choice(ld, size=300, replace=False)] = (np.float32(1.75) + rng.random(300, dtype=np.float32) * np.float32(0.25))
    rows.append(r); want.append(True)
    for extra, w in ((k - sp.size, True), (k - 1 - sp.size, False)):               # exactly k at the bound / k - 1
        r = np.full(ld, -5.0, np.float32)
        r[sp] = 5.0
        r[rng.choice(np.setdiff1d(np.arange(ld), sp), size=extra, replace=False)] = 5.0
        rows.append(r); want.append(w)
    scores = np.stack(rows)
    lengths = np.full(len(rows), ld, np.int32)
    for i, (row, w) in enumerate(zip(rows, want)):
        assert _takes_list_path(row, ld, k) == w, i
    _check(gpu_lib, scores, lengths, k, "sampled bound, both paths")


@pytest.mark.parametrize("k", [1, 64, 512, 2048])
def test_topk_sample_size_edges(gpu_lib, k):
    """Lengths where the sample reaches its minimum size (12544 = 3 * 4160 + 64
    positions), just below it, and where k is too large a share of the row for
    the bound to pay; bf16-rounded scores (many ties)."""
    rng = np.random.default_rng(7600 + k)
    ld = 20000
    lens = np.array([12543, 12544, 12545, 16383, 16384, 16385, 20000, 4160 * 4 + 63, 4160 * 4 + 64], np.int32)
    scores = wl.indexer_scores(rng, lens.size, ld, "bf16")
    paths = [_takes_list_path(scores[i], int(n), k) for i, n in enumerate(lens)]
    if k <= 512:
        assert not paths[0] and paths[1] and all(paths[1:]), paths
    _check(gpu_lib, scores, lens, k, f"sample size edges k={k}")


@pytest.mark.parametrize("k", [8191, 8192, 9000])
def test_topk_k_at_and_past_the_list(gpu_lib, k):
    """Full-length rows with k at the list's capacity (8192) and past it: the
    list path can take a row only if exactly k keys reach the bound, so these
    rows mostly count every key; lengths mixed."""
    rng = np.random.default_rng(7700 + k)
    ld, R = 65536, 8
    scores = wl.indexer_scores(rng, R, ld, "bf16")
    lengths = np.array([ld, ld - 1, 40000, 20000, k, k - 1, k + 1, 12544], np.int32)
    _check(gpu_lib, scores, lengths, k, f"k={k} near the list size")
