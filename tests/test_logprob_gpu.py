"""GPU parity and invariance of tig_logprob_gather (fused LM-head logprob).

[BitRL, section 2]: the logprob of every sampled token must be bit-identical
whatever the batch composition, the row position and the prefill / decode
split (diff = 0: max, mean, std of |delta| and k3 KL all exactly zero).
Parity bar against the fp64 oracle: |delta logprob| <= 1e-3 absolute.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bitwise, dev_bf16, diff_stats, record, say

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _parity(lp, lse, ref_lp, ref_lse, what):
    lp = lp.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    e1 = np.max(np.abs(lp - ref_lp))
    e2 = np.max(np.abs(lse - ref_lse))
    say(f"{what}: max |dlogprob| {e1:.3e}  max |dlse| {e2:.3e}")
    record("oracle_logprob", what, rows=int(lp.size), max_abs_logprob=float(e1), max_abs_lse=float(e2), bound=TOL)
    assert e1 <= TOL and e2 <= TOL, what
    return e1


def _tiny():
    cfg = wl.CONFIGS["tiny"]
    s = wl.streams(cfg.seed)
    H = wl.normal_bf16(s["H"], (max(cfg.M), cfg.K), 1.0)
    W = wl.normal_bf16(s["W"], (cfg.N, cfg.K), 0.02)
    ids = wl.uniform_ids(s["ids"], max(cfg.M), cfg.N)
    return cfg, H, W, ids


def test_tiny_every_M_parity_and_invariance(gpu_lib):
    cfg, H, W, ids = _tiny()
    Hd, Wd, idd = dev_bf16(H), dev_bf16(W), torch.from_numpy(ids).cuda()
    ref_lp, ref_lse = oracle.logprob_ref(H, W, ids)
    full_lp, full_lse = gpu_lib.logprob_gather(Hd, Wd, idd, cfg.leaves)
    _parity(full_lp, full_lse, ref_lp, ref_lse, "tiny M=64")
    for M in cfg.M:
        lp, lse = gpu_lib.logprob_gather(Hd[:M], Wd, idd[:M], cfg.leaves)
        assert_bitwise(lp, full_lp[:M], f"tiny logprob M={M}")
        assert_bitwise(lse, full_lse[:M], f"tiny lse M={M}")


@pytest.mark.parametrize("V", [1, 2, 127, 128, 129, 255, 1000, 4097])
@pytest.mark.parametrize("M", [1, 127, 128, 129, 300])
def test_tile_edges_parity(gpu_lib, M, V):
    rng = np.random.default_rng(M * 100003 + V)
    K = 512
    H = wl.normal_bf16(rng, (M, K), 1.0)
    W = wl.normal_bf16(rng, (V, K), 0.05)
    ids = rng.integers(0, V, size=M)
    lp, lse = gpu_lib.logprob_gather(dev_bf16(H), dev_bf16(W), torch.from_numpy(ids).cuda(), 8)
    ref_lp, ref_lse = oracle.logprob_ref(H, W, ids)
    _parity(lp, lse, ref_lp, ref_lse, f"M={M} V={V}")


@pytest.mark.parametrize("V", [4096, 151936, 1000, 129])
def test_equal_logits_closed_form(gpu_lib, V):
    """All W rows equal -> all logits equal -> logprob = -ln V (sum exp = V exactly)."""
    rng = np.random.default_rng(V)
    K = 512
    H = wl.normal_bf16(rng, (70, K), 1.0)
    row = wl.normal_bf16(rng, (1, K), 0.05)
    W = np.repeat(row, V, axis=0)
    ids = rng.integers(0, V, size=70)
    lp, lse = gpu_lib.logprob_gather(dev_bf16(H), dev_bf16(W), torch.from_numpy(ids).cuda(), 8)
    lp = lp.cpu().double().numpy()
    assert np.max(np.abs(lp + math.log(V))) < 1e-5
    # the logits themselves are the tree contraction's
    X = gpu_lib.tree_gemm(dev_bf16(H), dev_bf16(row), 8).cpu().double().numpy()[:, 0]
    assert np.max(np.abs(lse.cpu().double().numpy() - (X + math.log(V)))) < 1e-5


@pytest.mark.parametrize("V,M", [(151936, 100), (151936, 300), (4097, 130), (129, 64), (4097, 200),
                                 (129, 400)])
def test_one_distinct_logit_closed_form(gpu_lib, V, M):
    """One vocabulary row gives logit a, every other row 0: logprob = a - ln(e^a + V - 1)
    for the sampled id of that row and -ln(e^a + V - 1) for any other (a closed form,
    independent of the oracle), through the single-row-of-tiles path (up to 192 rows)
    and the multi-row one (at the full vocabulary and at ragged ones), with the
    distinct row in a middle tile and ids on both sides."""
    K, L = 1024, 8
    rng = np.random.default_rng(V + M)
    j = V // 2 + 3 if V > 8 else 0
    H = np.zeros((M, K), dtype=np.float32)
    Wf = np.zeros((V, K), dtype=np.float32)
    a_vals = np.array([0.5, 1.0, 2.0, 3.0, 5.5, 7.25, -1.5, 0.0])   # a = h * w, exact in bf16 and FP32
    h = a_vals[np.arange(M) % len(a_vals)]
    H[:, 17] = h                       # row m: logit a_m at column j, 0 elsewhere
    Wf[j, 17] = 1.0
    ids = np.where(np.arange(M) % 2 == 0, j, rng.integers(0, V, size=M))
    lp, lse = gpu_lib.logprob_gather(dev_bf16(wl.f32_to_bf16_bits(H)), dev_bf16(wl.f32_to_bf16_bits(Wf)),
                                     torch.from_numpy(ids).cuda(), L)
    lp = lp.cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    exp_lse = np.log(np.exp(h) + (V - 1))
    exp_lp = np.where(ids == j, h, 0.0) - exp_lse
    say(f"one distinct logit V={V} M={M}: max |dlogprob| {np.max(np.abs(lp - exp_lp)):.2e}")
    assert np.max(np.abs(lse - exp_lse)) < 1e-5
    assert np.max(np.abs(lp - exp_lp)) < 1e-5


# Vocabularies above 256 x 8 x 128 = 262144 tokens give the combine pass more
# than 8 vocabulary tiles per thread: it reads each row's tile partials twice
# (once for the max, once for the sum) instead of keeping them in registers.
@pytest.mark.parametrize("V", [262145, 1000003, 1 << 23])
def test_large_vocab_equal_logits_closed_form(gpu_lib, V):
    """All W rows equal: logprob = -ln V and lse = logit + ln V (the tile sums are
    exact, V < 2^24), and each row the same bits at every M."""
    K, L, Mmax = 512, 8, 37
    rng = np.random.default_rng(V)
    H = dev_bf16(wl.normal_bf16(rng, (Mmax, K), 1.0))
    row = dev_bf16(wl.normal_bf16(rng, (1, K), 0.05))
    W = row.expand(V, K).contiguous()
    ids = torch.from_numpy(rng.integers(0, V, size=Mmax)).cuda()
    say(f"equal logits V={V}")
    lp, lse = gpu_lib.logprob_gather(H, W, ids, L)
    x = gpu_lib.tree_gemm(H, row, L)[:, 0].double()
    assert float((lp.double() + math.log(V)).abs().max()) < 2e-5
    assert float((lse.double() - (x + math.log(V))).abs().max()) < 2e-5
    for M in (1, 2, 5, 36):
        a, b = gpu_lib.logprob_gather(H[:M], W, ids[:M], L)
        assert_bitwise(a, lp[:M], f"V={V} logprob M={M}")
        assert_bitwise(b, lse[:M], f"V={V} lse M={M}")


def test_large_vocab_parity(gpu_lib):
    """Random weights at a vocabulary of 1000003 (7813 tiles: the combine's
    re-read path, a last tile of 3 columns) against the fp64 oracle, and each
    row's bits independent of M."""
    K, V, L, M = 512, 1000003, 8, 6
    rng = np.random.default_rng(99)
    H = wl.normal_bf16(rng, (M, K), 1.0)
    W = wl.normal_bf16(rng, (V, K), 0.05)
    ids = rng.integers(0, V, size=M)
    ids[0], ids[1] = V - 1, 0
    Hd, Wd, idd = dev_bf16(H), dev_bf16(W), torch.from_numpy(ids).cuda()
    lp, lse = gpu_lib.logprob_gather(Hd, Wd, idd, L)
    ref_lp, ref_lse = oracle.logprob_ref(H, W, ids)
    _parity(lp, lse, ref_lp, ref_lse, f"V={V} M={M}")
    a, b = gpu_lib.logprob_gather(Hd[:1], Wd, idd[:1], L)
    assert_bitwise(a, lp[:1], "V=1000003 logprob M=1")
    assert_bitwise(b, lse[:1], "V=1000003 lse M=1")


def test_vocab_of_one(gpu_lib):
    """V = 1: lse is the single logit bit for bit and the logprob is exactly 0."""
    rng = np.random.default_rng(1)
    H = wl.normal_bf16(rng, (200, 512), 1.0)
    W = wl.normal_bf16(rng, (1, 512), 0.05)
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    lp, lse = gpu_lib.logprob_gather(Hd, Wd, torch.zeros(200, dtype=torch.int64, device="cuda:0"), 8)
    assert torch.all(lp == 0.0)
    assert_bitwise(lse, gpu_lib.tree_gemm(Hd, Wd, 8)[:, 0], "lse == logit")


def test_invalid_ids_give_nan_for_that_row_only(gpu_lib):
    cfg, H, W, ids = _tiny()
    ids = ids[:6].copy()
    ids[1], ids[4] = -1, cfg.N
    lp, lse = gpu_lib.logprob_gather(dev_bf16(H[:6]), dev_bf16(W), torch.from_numpy(ids).cuda(), 8)
    lp = lp.cpu().numpy()
    assert np.isnan(lp[1]) and np.isnan(lp[4])
    assert np.all(np.isfinite(lp[[0, 2, 3, 5]]))
    assert torch.all(torch.isfinite(lse))
    ref, _ = oracle.logprob_ref(H[:6], W, ids)
    assert np.max(np.abs(lp[[0, 2, 3, 5]] - ref[[0, 2, 3, 5]])) <= TOL


def test_lse_optional_and_repeatable(gpu_lib):
    cfg, H, W, ids = _tiny()
    Hd, Wd, idd = dev_bf16(H), dev_bf16(W), torch.from_numpy(ids).cuda()
    a, _ = gpu_lib.logprob_gather(Hd, Wd, idd, 8, with_lse=False)
    for _ in range(5):
        b, _ = gpu_lib.logprob_gather(Hd, Wd, idd, 8)
        assert_bitwise(a, b, "repeat / lse optional")


def _prefill_decode(gpu_lib, name, n_oracle_rows, shuffle):
    cfg = wl.CONFIGS[name]
    s = wl.streams(cfg.seed)
    M = cfg.n_seq * cfg.n_pos
    say(f"{name}: generating H[{M},{cfg.K}] W[{cfg.N},{cfg.K}]")
    H = wl.normal_bf16(s["H"], (M, cfg.K), 1.0)
    W = wl.normal_bf16(s["W"], (cfg.N, cfg.K), 0.02)
    ids = wl.uniform_ids(s["ids"], M, cfg.N)
    # rows checked against the oracle take ids drawn from the softmax itself
    rows = np.sort(s["perm"].choice(M, size=n_oracle_rows, replace=False))
    W64 = oracle.bf16_bits_to_f64(W)
    X = oracle.contraction_ref(H[rows], W64)
    ids[rows] = oracle.gumbel_max_ids(X, wl.gumbel(s["gumbel"], X.shape))
    ref_lp, ref_lse = oracle.logprob_ref(H[rows], W64, ids[rows])
    del X, W64

    Hd, Wd, idd = dev_bf16(H), dev_bf16(W), torch.from_numpy(ids).cuda()
    prefill_rows, steps = wl.prefill_decode_rows(cfg.n_seq, cfg.n_pos, s["extra"] if shuffle else None)
    say(f"{name}: prefill M={M}")
    lp, lse = gpu_lib.logprob_gather(Hd, Wd, idd, cfg.leaves)
    _parity(lp[rows], lse[rows], ref_lp, ref_lse, f"{name} sampled rows vs oracle")
    say(f"{name}: {cfg.n_pos} decode steps of {cfg.n_seq}")
    dec_lp = torch.empty_like(lp)
    dec_lse = torch.empty_like(lse)
    ws = torch.empty(gpu_lib.tig_logprob_workspace_bytes(cfg.n_seq, cfg.K, cfg.N, cfg.leaves),
                     dtype=torch.uint8, device="cuda:0")
    for t in range(cfg.n_pos):
        r = torch.from_numpy(steps[t]).cuda()
        a, b = gpu_lib.logprob_gather(Hd[r].contiguous(), Wd, idd[r].contiguous(), cfg.leaves, workspace=ws)
        dec_lp[r] = a
        dec_lse[r] = b
    st = diff_stats(lp.cpu().numpy(), dec_lp.cpu().numpy())
    say(f"{name}: prefill vs decode diff {st}")
    assert_bitwise(dec_lp, lp, f"{name} prefill vs decode logprob")
    assert_bitwise(dec_lse, lse, f"{name} prefill vs decode lse")
    assert st == {"max": 0.0, "mean": 0.0, "std": 0.0, "k3": 0.0}


@pytest.mark.slow
def test_lmhead_prefill_vs_decode(gpu_lib):
    _prefill_decode(gpu_lib, "lmhead", n_oracle_rows=256, shuffle=False)


@pytest.mark.slow
def test_large_prefill_vs_decode(gpu_lib):
    _prefill_decode(gpu_lib, "large", n_oracle_rows=128, shuffle=True)
