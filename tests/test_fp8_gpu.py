"""GPU parity of block-FP8 quantisation and the W8A8 leaf-tree GEMM.

[BitRL, section 4.1]: BF16 master weights are quantised to block FP8 by the
deployment rule and the product runs W8A8, with one accumulation order for
every M; [BitRL, section 4.4]: the FP8 inputs are rounded per element to
nearest.  Quantisation is integer-exact: codes and scales must equal the
oracle's bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bitwise, assert_gemm_close, dev_bf16, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _special(X, rng):
    """Blocks that test the exponent rule's edges, in bf16 bits."""
    X = X.copy()
    one = wl.f32_to_bf16_bits(np.float32(1.0))
    X[0, :128] = 0                                                      # all-zero block: e = 0
    X[1, :128] = wl.f32_to_bf16_bits(np.float32(448.0))                 # amax exactly 448: e = 0
    X[2, :64] = wl.f32_to_bf16_bits(np.float32(1.75))                   # amax 1.75: e = -8 exactly
    X[2, 64:128] = one
    X[3, :128] = wl.f32_to_bf16_bits((rng.standard_normal(128) * 1e-30).astype(np.float32))   # tiny
    X[4, :128] = 0x8000                                                 # -0 everywhere
    X[5, 5] = wl.f32_to_bf16_bits(np.array([-3.3895e38], np.float32))[0]   # largest bf16 magnitude
    return X


@pytest.mark.parametrize("block_rows,R,C", [(1, 77, 1000), (1, 6, 128), (1, 9, 130), (1, 7, 384),
                                            (128, 300, 260), (128, 128, 384), (128, 130, 130)])
def test_fp8_quantize_bitwise(gpu_lib, block_rows, R, C):
    rng = np.random.default_rng(4000 + R + C)
    X = _special(wl.normal_bf16(rng, (R, C), 0.5 if block_rows == 1 else 0.02), rng)
    say(f"fp8 quantize block_rows={block_rows} R={R} C={C}")
    Q, S = gpu_lib.fp8_quantize(dev_bf16(X), block_rows)
    q_ref, e_ref = oracle.fp8_block_quant(X, block_rows, 128)
    assert np.array_equal(Q.cpu().numpy(), q_ref)
    assert np.array_equal(S.cpu().numpy().astype(np.int64) - 127, e_ref)


def test_fp8_quantize_strided_rows(gpu_lib):
    rng = np.random.default_rng(4100)
    X = wl.normal_bf16(rng, (40, 300), 1.0)
    Xd = dev_bf16(X)[:, :260]                                           # row stride 300, 260 columns
    Q, S = gpu_lib.fp8_quantize(Xd, 1)
    q_ref, e_ref = oracle.fp8_block_quant(X[:, :260], 1, 128)
    assert np.array_equal(Q.cpu().numpy(), q_ref) and np.array_equal(S.cpu().numpy().astype(np.int64) - 127, e_ref)


def _quant_pair(gpu_lib, A, W):
    QA, SA = gpu_lib.fp8_quantize(dev_bf16(A), 1)
    QW, SW = gpu_lib.fp8_quantize(dev_bf16(W), 128)
    return QA, SA, QW, SW


@pytest.mark.parametrize("M,N,K,L", [(257, 300, 1024, 8), (1, 130, 1024, 8), (64, 256, 2048, 16),
                                     (300, 129, 512, 1), (129, 640, 4096, 4)])
def test_fp8_gemm_matches_oracle(gpu_lib, M, N, K, L):
    rng = np.random.default_rng(4200 + M + N + K)
    A = wl.normal_bf16(rng, (M, K), 1.0)
    W = wl.normal_bf16(rng, (N, K), 0.02)
    say(f"fp8 gemm M={M} N={N} K={K} L={L}")
    QA, SA, QW, SW = _quant_pair(gpu_lib, A, W)
    C = gpu_lib.fp8_tree_gemm(QA, SA, QW, SW, L)
    qa, qw = QA.cpu().numpy(), QW.cpu().numpy()
    ea, ew = SA.cpu().numpy().astype(np.int64) - 127, SW.cpu().numpy().astype(np.int64) - 127
    ref = oracle.fp8_gemm_ref(qa, ea, qw, ew)
    worst = assert_gemm_close(C.cpu().numpy(), ref, what="fp8 gemm")
    say(f"fp8 gemm worst relative error {worst:.3e}")
    # the same product through the bf16 matrix cores (exact operands, another order)
    Ad = gpu_lib.fp8_dequantize(QA, SA, 1)
    Wd = gpu_lib.fp8_dequantize(QW, SW, 128)
    assert_gemm_close(gpu_lib.tree_gemm(Ad, Wd, L).cpu().numpy(), ref, what="bf16 path of the same values")
    Cb = gpu_lib.fp8_tree_gemm(QA, SA, QW, SW, L, torch.bfloat16)
    assert np.array_equal(Cb.cpu().view(torch.int16).numpy().view(np.uint16), wl.f32_to_bf16_bits(C.cpu().numpy()))


def test_fp8_dequantize_is_exact(gpu_lib):
    rng = np.random.default_rng(4250)
    for br, (R, C) in ((1, (50, 384)), (128, (200, 260))):
        X = _special(wl.normal_bf16(rng, (R, C), 0.3), rng)
        Q, S = gpu_lib.fp8_quantize(dev_bf16(X), br)
        D = gpu_lib.fp8_dequantize(Q, S, br).cpu().view(torch.int16).numpy().view(np.uint16)
        ref = oracle.fp8_dequant(Q.cpu().numpy(), S.cpu().numpy().astype(np.int64) - 127, br)
        # exact in bf16, except a largest-magnitude value that rounded up to 2^8 * 2^120 = 2^128,
        # which overflows to an infinity: compare with the rounding of the exact value
        assert np.array_equal(D, oracle.f64_to_bf16_rne(ref))


def _codes(vals):
    """E4M3 codes of exactly representable values."""
    return oracle.f64_to_e4m3_rne(np.asarray(vals, dtype=np.float64))


def test_fp8_gemm_exact_on_integer_products(gpu_lib):
    """Small integer values (codes of -4 .. 4, scales 1): every product and
    partial sum is an integer far below 2^24, so any order gives the exact sum."""
    rng = np.random.default_rng(4260)
    M, N, K, L = 200, 260, 1024, 8
    qa = _codes(rng.integers(-4, 5, size=(M, K)))
    qw = _codes(rng.integers(-4, 5, size=(N, K)))
    SA = torch.full((M, K // 128), 127, dtype=torch.uint8, device=DEV)
    SW = torch.full((-(-N // 128), K // 128), 127, dtype=torch.uint8, device=DEV)
    C = gpu_lib.fp8_tree_gemm(torch.from_numpy(qa).to(DEV), SA, torch.from_numpy(qw).to(DEV), SW, L)
    exact = oracle.e4m3_value(qa).astype(np.int64) @ oracle.e4m3_value(qw).astype(np.int64).T
    assert np.array_equal(C.cpu().numpy().astype(np.int64), exact)


def test_fp8_gemm_leaf_tree_closed_form(gpu_lib):
    """K = 8 leaves of 128; leaf partials 2^24 (one product 2^12 * 2^12 through the
    scales) and seven 1s (1 * 1).  The balanced tree gives ((2^24 + 1) + 2) + 4 =
    2^24 + 6 (2^24 + 1 ties to 2^24); a sequential sum gives 2^24, the exact sum
    2^24 + 7.  The large leaf sits at every position in turn."""
    L, K, N = 8, 1024, 128
    M = L
    qa = np.zeros((M, K), np.uint8)
    qw = np.zeros((N, K), np.uint8)
    one = int(_codes([1.0])[0])
    ea = np.zeros((M, K // 128), np.int64)
    ew = np.zeros((1, K // 128), np.int64)
    for r in range(M):
        for leaf in range(L):
            qa[r, leaf * 128] = one
            if leaf == r:
                ea[r, leaf] = 12
    qw[:, :] = 0
    qw[:, ::128] = one
    ew[0, :] = 12
    # W's scale applies to all rows: undo it on the small leaves through A's scale
    for r in range(M):
        for leaf in range(L):
            if leaf != r:
                ea[r, leaf] = -12
    C = gpu_lib.fp8_tree_gemm(torch.from_numpy(qa).to(DEV), torch.from_numpy((ea + 127).astype(np.uint8)).to(DEV),
                              torch.from_numpy(qw).to(DEV), torch.from_numpy((ew + 127).astype(np.uint8)).to(DEV),
                              L).cpu().numpy()
    assert np.all(C == np.float32(2.0 ** 24 + 6)), np.unique(C)


def test_fp8_repeat_calls_identical(gpu_lib):
    rng = np.random.default_rng(4280)
    A = wl.normal_bf16(rng, (700, 2048), 1.0)
    W = wl.normal_bf16(rng, (520, 2048), 0.02)
    QA, SA, QW, SW = _quant_pair(gpu_lib, A, W)
    first = gpu_lib.fp8_tree_gemm(QA, SA, QW, SW, 8)
    for _ in range(3):
        assert_bitwise(gpu_lib.fp8_tree_gemm(QA, SA, QW, SW, 8), first, "fp8 gemm repeat")
        Q2, S2 = gpu_lib.fp8_quantize(dev_bf16(A), 1)
        assert torch.equal(Q2, QA) and torch.equal(S2, SA)


def test_fp8_path_rows_do_not_depend_on_the_batch(gpu_lib):
    """Quantise + GEMM of a row alone equals the same row inside batches of
    several sizes (per-token activation blocks, one accumulation order)."""
    rng = np.random.default_rng(4300)
    K, N, L = 1024, 384, 8
    A = wl.normal_bf16(rng, (300, K), 1.0)
    W = wl.normal_bf16(rng, (N, K), 0.02)
    QW, SW = gpu_lib.fp8_quantize(dev_bf16(W), 128)
    full = None
    for M in (300, 193, 64, 1):
        QA, SA = gpu_lib.fp8_quantize(dev_bf16(A[:M]), 1)
        C = gpu_lib.fp8_tree_gemm(QA, SA, QW, SW, L)
        if full is None:
            full = C
        else:
            assert_bitwise(C, full[:M], f"fp8 rows of a {M}-row batch")


@pytest.mark.slow
def test_fp8_linear_config(gpu_lib):
    """The linear config (4097 x 4096 x 4096, 8 leaves): sampled rows against the oracle."""
    cfg = wl.CONFIGS["linear"]
    s = wl.streams(cfg.seed)
    A = wl.normal_bf16(s["H"], (4097, cfg.K), 1.0)
    W = wl.normal_bf16(s["W"], (cfg.N, cfg.K), 0.02)
    QA, SA, QW, SW = _quant_pair(gpu_lib, A, W)
    C = gpu_lib.fp8_tree_gemm(QA, SA, QW, SW, cfg.leaves).cpu().numpy()
    rows = np.concatenate([[0, 4095, 4096], s["perm"].choice(4097, 61, replace=False)])
    qa, qw = QA.cpu().numpy(), QW.cpu().numpy()
    ea, ew = SA.cpu().numpy().astype(np.int64) - 127, SW.cpu().numpy().astype(np.int64) - 127
    ref = oracle.fp8_gemm_ref(qa[rows], ea[rows], qw, ew)
    assert_gemm_close(C[rows], ref, what="fp8 linear config")
    q_ref, e_ref = oracle.fp8_block_quant(A[rows], 1, 128)
    assert np.array_equal(qa[rows], q_ref) and np.array_equal(ea[rows], e_ref)
