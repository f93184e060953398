"""Schedule freedom on the GPU: tile height, leaf visiting order, sampled-logit pass.

The dense kernels use 192-row tiles where that needs fewer tiles than 128-row
ones (and 128 rows otherwise; tree_gemm takes 64, 128 or 192 rows, whichever
lets its busiest workgroup finish first, and at most 128 at 16 leaves, while the logprob
path then keeps the left half of each tile's leaf tree in scratch and adds it
to the right half's root at the end), and a workgroup that runs several tiles
visits the leaves of every other tile last to first.  Only the schedule may
depend on these choices: a row's bits must not [BitRL, section 2: one
accumulation order for every M].  The sampled token's logit is
computed by its own pass with the same MFMA k-steps and leaf tree, so logprob
must equal the FP32 difference of the contraction's own element and the
log-sum-exp, bit for bit.
"""

from fractions import Fraction

from test_oracle_pins import load_golden, parse_dyadic

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_bitwise, dev_bf16, say

pytestmark = pytest.mark.gpu


def _busiest(n_mt, n_nt, cus):
    """Tiles of the busiest workgroup under the persistent deal (one workgroup
    per CU in groups of 8 XCDs; n-slices per XCD from 32 n-tiles up)."""
    tiles = n_mt * n_nt
    slots = min(-(-tiles // 8) * 8, max(cus // 8 * 8, 8)) // 8
    per_xcd = -(-n_nt // 8) * n_mt if n_nt >= 32 else -(-tiles // 8)
    return -(-per_xcd // slots)


def _block_m(M, L, logprob=False, N=None):
    if logprob:
        return 192 if -(-M // 192) < -(-M // 128) else 128
    # tree_gemm: the height whose busiest workgroup finishes first, by the
    # relative tile times 70 / 100 / 138 of 64 / 128 / 192 rows.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    heights = (64, 128, 192) if L <= 8 else (64, 128)
    cost = {64: 70, 128: 100, 192: 138}
    return min(heights, key=lambda h: _busiest(-(-M // h), -(-N // 128), cus) * cost[h])


# (start, stop) slices of a 577-row batch at different row offsets.  logprob:
# 128-row tiles for M <= 128 and M = 256, 192-row tiles for 129, 177, 512 and
# 577 rows; tree_gemm over 64 n-tiles: 64-row tiles up to 256 rows, 128-row
# tiles for 512 rows, 192 rows for 577 up to 8 leaves (128 at 16).
SLICES = [(0, 1), (0, 128), (100, 229), (400, 577), (33, 289), (40, 552), (0, 577)]


@pytest.mark.parametrize("L", [1, 8, 16])
def test_logprob_rows_identical_across_tile_heights(gpu_lib, L):
    K, V, M = 1024, 1000, 577
    rng = np.random.default_rng(4242 + L)
    H = dev_bf16(wl.normal_bf16(rng, (M, K), 1.0))
    W = dev_bf16(wl.normal_bf16(rng, (V, K), 0.02))
    ids = torch.from_numpy(rng.integers(0, V, size=M)).to("cuda:0")
    full_lp, full_lse = gpu_lib.logprob_gather(H, W, ids, L)
    heights = set()
    for a, b in SLICES:
        heights.add(_block_m(b - a, L, logprob=True))
        say(f"logprob L={L} rows [{a}, {b}) tile rows {_block_m(b - a, L, logprob=True)}")
        lp, lse = gpu_lib.logprob_gather(H[a:b].contiguous(), W, ids[a:b].contiguous(), L)
        assert_bitwise(lp, full_lp[a:b], f"logprob rows [{a},{b}) L={L}")
        assert_bitwise(lse, full_lse[a:b], f"lse rows [{a},{b}) L={L}")
    assert heights == {128, 192}


@pytest.mark.parametrize("L", [2, 8, 16])
def test_tree_gemm_rows_identical_across_tile_heights(gpu_lib, L):
    """64 columns of n-tiles: the slices run on 64-, 128- and 192-row tiles
    (only 64 and 128 at 16 leaves); the last columns (N = 8187) leave a ragged
    n-tile; a narrow W (300 columns) puts the whole batch on 64-row tiles."""
    K, N, M = 1024, 8187, 577
    rng = np.random.default_rng(777 + L)
    A = dev_bf16(wl.normal_bf16(rng, (M, K), 1.0))
    W = dev_bf16(wl.normal_bf16(rng, (N, K), 0.02))
    full = gpu_lib.tree_gemm(A, W, L)
    narrow = gpu_lib.tree_gemm(A, W[:300].contiguous(), L)
    assert_bitwise(narrow, full[:, :300], f"tree_gemm narrow W L={L}")
    heights = {_block_m(M, L, N=300)}
    for a, b in SLICES:
        h = _block_m(b - a, L, N=N)
        heights.add(h)
        say(f"tree_gemm L={L} rows [{a}, {b}) tile rows {h}")
        part = gpu_lib.tree_gemm(A[a:b].contiguous(), W, L)
        assert_bitwise(part, full[a:b], f"tree_gemm rows [{a},{b}) L={L}")
    assert heights == ({64, 128, 192} if L <= 8 else {64, 128})


@pytest.mark.parametrize("L", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("M", [5, 150, 577])
def test_picked_logit_is_the_contraction_element(gpu_lib, L, M):
    K, V = 2048, 777
    rng = np.random.default_rng(M * 31 + L)
    H = dev_bf16(wl.normal_bf16(rng, (M, K), 1.0))
    W = dev_bf16(wl.normal_bf16(rng, (V, K), 0.02))
    ids_np = rng.integers(0, V, size=M)
    ids = torch.from_numpy(ids_np).to("cuda:0")
    say(f"picked logit M={M} L={L}")
    lp, lse = gpu_lib.logprob_gather(H, W, ids, L)
    C = gpu_lib.tree_gemm(H, W, L).cpu().numpy()
    x = C[np.arange(M), ids_np].astype(np.float32)
    expect = (x - lse.cpu().numpy().astype(np.float32)).astype(np.float32)
    assert_bitwise(lp, torch.from_numpy(expect), f"logprob vs C[row, id] - lse (M={M}, L={L})")


# More tiles than workgroups (one per CU), so workgroups run a second, odd tile
# whose leaves they visit last to first.
MANY = {8: (2048, 4224, 512), 16: (2048, 4224, 1024)}


@pytest.mark.parametrize("L", [8, 16])
def test_many_tiles_tree_closed_form(gpu_lib, L):
    golden = {r[0]: r for r in load_golden("tree_f32_closed_forms.txt")}
    key = "L8_adjacent" if L == 8 else "L16_adjacent"
    vals = [parse_dyadic(v) for v in golden[key][1].split(",")]
    expect = parse_dyadic(golden[key][2])
    M, N, K = MANY[L]
    say(f"many tiles closed form M={M} N={N} K={K} L={L}")
    ell = K // L
    A = np.zeros((M, K), dtype=np.float32)
    W = np.zeros((N, K), dtype=np.float32)
    scale = np.array([float(Fraction(2) ** -(n % 7)) for n in range(N)])
    for l in range(L):
        A[:, l * ell] = 1.0
        W[:, l * ell] = float(vals[l]) * scale
    C = gpu_lib.tree_gemm(dev_bf16(wl.f32_to_bf16_bits(A)), dev_bf16(wl.f32_to_bf16_bits(W)), L)
    exp = np.array([float(expect * Fraction(2) ** -(n % 7)) for n in range(N)], dtype=np.float32)
    assert_bitwise(C, torch.from_numpy(np.tile(exp, (M, 1))), "tree closed form, many tiles")


@pytest.mark.parametrize("L", [8, 16])
def test_many_tiles_rows_match_single_row_calls(gpu_lib, L):
    M, N, K = MANY[L]
    rng = np.random.default_rng(99 + L)
    A = dev_bf16(wl.normal_bf16(rng, (M, K), 1.0))
    W = dev_bf16(wl.normal_bf16(rng, (N, K), 0.02))
    ids = torch.from_numpy(rng.integers(0, N, size=M)).to("cuda:0")
    say(f"many tiles M={M} N={N} K={K} L={L}: batch")
    C = gpu_lib.tree_gemm(A, W, L)
    lp, lse = gpu_lib.logprob_gather(A, W, ids, L)
    for r in np.linspace(0, M - 1, 12).astype(int):
        c1 = gpu_lib.tree_gemm(A[r:r + 1].contiguous(), W, L)
        assert_bitwise(c1, C[r:r + 1], f"tree_gemm row {r} alone vs in the batch (L={L})")
        l1, s1 = gpu_lib.logprob_gather(A[r:r + 1].contiguous(), W, ids[r:r + 1].contiguous(), L)
        assert_bitwise(l1, lp[r:r + 1], f"logprob row {r} alone vs in the batch (L={L})")
        assert_bitwise(s1, lse[r:r + 1], f"lse row {r} alone vs in the batch (L={L})")
