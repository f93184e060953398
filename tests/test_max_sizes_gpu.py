"""GPU: the longest contraction the boundary accepts.

tig_tree_gemm and tig_logprob_gather take K up to where 192 rows of the bf16
operand would span 2 GiB: K = 5592064, the largest multiple of 8 x 64 below
2^31 / 384, and also a multiple of 16 x 64.  The inputs are random
signs times powers of two (H and A: +-1, W: +-2^-12), so every product is
+-2^-12 and every partial sum an integer multiple of 2^-12 below 2^24 of them
in magnitude: the FP32 leaf sums and the tree are exact whatever their order,
the contraction is compared bit for bit with the oracle's exact value, and the
logprob to the oracle's 1e-3 ([BitRL, section 2]).  The oracle's contraction
runs over K in chunks only to bound host memory; with these inputs every
chunk sum and their total are exact in float64, so the chunking changes no
value.  A 192-row logprob call runs as one row of 192-row tiles, whose last
row starts 2.1 GB past the first; its rows are also called alone and in the
first 128 and must keep their bits.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bitwise, dev_bf16, record, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

K = 5592064     # 2^31 / (192 * 2) rounded down to a multiple of 8 * 64; also a multiple of 16 * 64
assert 192 * K * 2 < 2 ** 31 <= 192 * (K + 512) * 2 and K % 1024 == 0
M, V = 192, 130
TOL = 1e-3
ROWS = np.array([0, 1, 63, 64, 127, 128, 129, 190, 191])


def _exact_contraction(A, W):
    """oracle.contraction_ref in column chunks."""
    out = np.zeros((A.shape[0], W.shape[0]), dtype=np.float64)
    step = 1 << 19
    for k0 in range(0, A.shape[1], step):
        k1 = min(A.shape[1], k0 + step)
        out += oracle.contraction_ref(np.ascontiguousarray(A[:, k0:k1]), np.ascontiguousarray(W[:, k0:k1]))
    return out


@pytest.fixture(scope="module")
def inputs():
    rng = np.random.default_rng(5592064)
    say(f"max-K inputs: H {M} x {K}, W {V} x {K} (random signs)")
    H = wl.sign_bf16(rng, (M, K), 0)
    W = wl.sign_bf16(rng, (V, K), -12)
    ids = wl.uniform_ids(rng, M, V)
    X = _exact_contraction(H[ROWS], W)
    Hd, Wd = dev_bf16(H), dev_bf16(W)
    del H, W
    return Hd, Wd, torch.from_numpy(ids).to("cuda:0"), ids, X


def test_tree_gemm_longest_k(gpu_lib, inputs):
    Hd, Wd, _, _, X = inputs
    say(f"tree GEMM {M} x {V} x {K}, 8 leaves")
    C = gpu_lib.tree_gemm(Hd, Wd, 8)
    assert np.all(np.abs(X) * 4096 < 2 ** 24)          # exact in FP32 at every step
    assert_bitwise(C[torch.from_numpy(ROWS).to(C.device)], torch.from_numpy(X.astype(np.float32)),
                   "longest-K contraction")


@pytest.mark.parametrize("L", [8, 16])
def test_logprob_longest_k_192_row_tile(gpu_lib, inputs, L):
    H, W, idd, ids, X = inputs
    say(f"logprob M={M} V={V} K={K} L={L}")
    ws = torch.empty(gpu_lib.tig_logprob_workspace_bytes(M, K, V, L), dtype=torch.uint8, device="cuda:0")
    lp = torch.empty(M, dtype=torch.float32, device="cuda:0")
    lse = torch.empty_like(lp)
    gpu_lib.tig_logprob_gather(H, W, idd, lp, lse, L, ws)
    ref_lse = oracle.lse_ref(X)
    ref_lp = oracle.log_softmax_ref(X)[np.arange(ROWS.size), ids[ROWS]]
    got_lp = lp.cpu().double().numpy()[ROWS]
    got_lse = lse.cpu().double().numpy()[ROWS]
    e1, e2 = np.max(np.abs(got_lp - ref_lp)), np.max(np.abs(got_lse - ref_lse))
    say(f"  max |dlogprob| {e1:.3e}  max |dlse| {e2:.3e}")
    record("oracle_logprob", f"longest K, {L} leaves", rows=int(ROWS.size), max_abs_logprob=float(e1),
           max_abs_lse=float(e2), bound=TOL)
    assert e1 <= TOL and e2 <= TOL
    # The same rows called alone (one row) and as the first 128 (a 128-row tile).
    for r0, r1 in ((191, 192), (0, 1), (0, 128), (129, 130)):
        a = torch.empty(r1 - r0, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        gpu_lib.tig_logprob_gather(H[r0:r1], W, idd[r0:r1], a, b, L, ws)
        assert_bitwise(a, lp[r0:r1], f"logprob rows {r0}..{r1 - 1} alone")
        assert_bitwise(b, lse[r0:r1], f"lse rows {r0}..{r1 - 1} alone")
