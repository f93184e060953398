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


@pytest.mark.parametrize("block_rows,R,C", [(1, 77, 1000), (1, 6, 128), (128, 300, 260), (128, 128, 384)])
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


@pytest.mark.parametrize("M,N,K,L", [(257, 300, 1024, 8), (1, 130, 512, 8), (64, 256, 2048, 16)])
def test_fp8_gemm_matches_oracle_and_is_the_dequantised_tree(gpu_lib, M, N, K, L):
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
    # the dequantised operands are exact bf16 values: the product is tig_tree_gemm on them
    Ad = wl.f32_to_bf16_bits(oracle.fp8_dequant(qa, ea, 1).astype(np.float32))
    Wd = wl.f32_to_bf16_bits(oracle.fp8_dequant(qw, ew, 128).astype(np.float32))
    assert np.array_equal(oracle.bf16_bits_to_f64(Ad), oracle.fp8_dequant(qa, ea, 1))
    assert_bitwise(C, gpu_lib.tree_gemm(dev_bf16(Ad), dev_bf16(Wd), L), "fp8 gemm vs tree_gemm of dequantised")
    Cb = gpu_lib.fp8_tree_gemm(QA, SA, QW, SW, L, torch.bfloat16)
    assert np.array_equal(Cb.cpu().view(torch.int16).numpy().view(np.uint16), wl.f32_to_bf16_bits(C.cpu().numpy()))


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
