"""GPU parity and invariance of tig_moe_tree_gemm_combine (MoE-shaped path).

[BitRL, 4.4]: an expert's result for a row must not depend on the layout the
row arrives in; [BitRL, 4.5] and [IsoExec, Parallelism-invariant kernels]: the
expert outputs are combined in FP32 in a fixed order (here: ascending expert
id, a float32 multiply then a float32 add).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bitwise, assert_gemm_close, dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    cfg = wl.CONFIGS["moe"]
    s = wl.streams(cfg.seed)
    H = wl.normal_bf16(s["H"], (cfg.tokens, cfg.K), 1.0)
    We = wl.normal_bf16(s["W"], (cfg.experts, cfg.N, cfg.K), 0.02)
    ids, w = wl.routing_input(s["route"], cfg.tokens, cfg.experts, cfg.topk)
    return cfg, H, We, ids, w, s["perm"]


def _run(gpu_lib, H, We, ids, w, L):
    return gpu_lib.moe_tree_gemm_combine(dev_bf16(H), dev_bf16(We), torch.from_numpy(ids).cuda(),
                                         torch.from_numpy(w).cuda(), L)


def test_moe_config_parity(gpu_lib, moe):
    cfg, H, We, ids, w, _ = moe
    say("moe parity: 4096 tokens, 64 experts 2048->1408, top-8")
    out = _run(gpu_lib, H, We, ids, w, cfg.leaves)
    ref = oracle.moe_ref(H, We, ids, w)
    worst = assert_gemm_close(out.cpu().numpy(), ref, what="moe")
    say(f"moe worst relative error {worst:.3e}")


def test_moe_split_and_permutation_invariance(gpu_lib, moe):
    cfg, H, We, ids, w, rng = moe
    Hd, Wd = dev_bf16(H), dev_bf16(We)
    idd, wd = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    full = gpu_lib.moe_tree_gemm_combine(Hd, Wd, idd, wd, cfg.leaves)
    say("moe: 32 calls of 128 tokens")
    parts = [gpu_lib.moe_tree_gemm_combine(Hd[i:i + 128], Wd, idd[i:i + 128], wd[i:i + 128], cfg.leaves)
             for i in range(0, cfg.tokens, 128)]
    assert_bitwise(torch.cat(parts), full, "moe 1 x 4096 vs 32 x 128")
    p = torch.from_numpy(rng.permutation(cfg.tokens)).cuda()
    perm = gpu_lib.moe_tree_gemm_combine(Hd[p].contiguous(), Wd, idd[p].contiguous(), wd[p].contiguous(),
                                         cfg.leaves)
    assert_bitwise(perm, full[p], "moe permuted tokens")
    # slot order does not matter: the combine runs in ascending expert id
    q = torch.from_numpy(rng.permutation(cfg.topk)).cuda()
    swapped = gpu_lib.moe_tree_gemm_combine(Hd, Wd, idd[:, q].contiguous(), wd[:, q].contiguous(), cfg.leaves)
    assert_bitwise(swapped, full, "moe slot order")


def test_moe_top1_unit_gate_is_tree_gemm(gpu_lib, moe):
    cfg, H, We, ids, w, _ = moe
    T = 1000
    ids1 = ids[:T, :1].copy()
    w1 = np.ones((T, 1), dtype=np.float32)
    out = _run(gpu_lib, H[:T], We, ids1, w1, cfg.leaves)
    Hd = dev_bf16(H[:T])
    for e in np.unique(ids1[:, 0])[:16]:
        rows = np.nonzero(ids1[:, 0] == e)[0]
        C = gpu_lib.tree_gemm(Hd, dev_bf16(We[e]), cfg.leaves)
        assert_bitwise(out[rows], C[rows], f"expert {e}")


def test_moe_integer_exact(gpu_lib):
    rng = np.random.default_rng(5)
    T, E, N, K, topk = 300, 8, 200, 512, 4
    H = wl.integer_bf16(rng, (T, K), -3, 3)
    We = wl.integer_bf16(rng, (E, N, K), -3, 3)
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    w = rng.choice(np.array([0.25, 0.5, 1.0, 2.0], dtype=np.float32), size=(T, topk))
    out = _run(gpu_lib, H, We, ids, w, 8)
    ref = oracle.moe_ref(H, We, ids, w).astype(np.float32)
    assert_bitwise(out, torch.from_numpy(ref), "integer MoE")


def test_moe_combine_order_matches_emulator(gpu_lib):
    """Exact expert outputs, arbitrary float32 gates: only the combine rounds."""
    rng = np.random.default_rng(6)
    T, E, N, K, topk = 257, 16, 130, 512, 8
    H = wl.integer_bf16(rng, (T, K), -2, 2)
    We = wl.integer_bf16(rng, (E, N, K), -2, 2)
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, topk)).astype(np.float32)
    out = _run(gpu_lib, H, We, ids, w, 8)
    Y = np.stack([oracle.contraction_ref(H, We[e]) for e in range(E)])      # [E, T, N], exact
    Yp = Y[ids, np.arange(T)[:, None]].astype(np.float32)                  # [T, topk, N]
    ref = oracle.moe_combine_f32(Yp, ids, w)
    assert_bitwise(out, torch.from_numpy(ref), "combine order")
    slot = np.zeros((T, N), dtype=np.float32)
    for s_ in range(topk):
        slot = np.add(slot, np.multiply(w[:, s_:s_ + 1], Yp[:, s_], dtype=np.float32), dtype=np.float32)
    assert np.any(slot != ref), "slot order should differ somewhere (power of the check)"


@pytest.mark.parametrize("N", [132, 130])
def test_moe_repeated_expert_keeps_slot_order(gpu_lib, N):
    """A token may route two slots to one expert: equal ids combine in slot order.

    Exact expert outputs and float32 gates make the combine the only rounding;
    N = 132 takes the four-column path of the combine, N = 130 the scalar one.
    """
    rng = np.random.default_rng(60 + N)
    T, E, K, topk = 97, 6, 512, 8
    H = wl.integer_bf16(rng, (T, K), -2, 2)
    We = wl.integer_bf16(rng, (E, N, K), -2, 2)
    ids = rng.integers(0, E, size=(T, topk)).astype(np.int32)   # repeats within a token
    assert any(len(set(r)) < topk for r in ids.tolist())
    w = rng.random((T, topk)).astype(np.float32)
    say(f"moe repeated experts N={N}")
    out = _run(gpu_lib, H, We, ids, w, 8)
    Y = np.stack([oracle.contraction_ref(H, We[e]) for e in range(E)])
    Yp = Y[ids, np.arange(T)[:, None]].astype(np.float32)
    ref = oracle.moe_combine_f32(Yp, ids, w)
    assert_bitwise(out, torch.from_numpy(ref), f"repeated experts, N={N}")


def test_moe_invalid_expert_gives_nan_for_that_token(gpu_lib):
    rng = np.random.default_rng(7)
    T, E, N, K, topk = 10, 4, 64, 512, 2
    H = wl.normal_bf16(rng, (T, K))
    We = wl.normal_bf16(rng, (E, N, K), 0.05)
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    ids[3, 1] = E
    ids[7, 0] = -2
    w = np.full((T, topk), 0.5, dtype=np.float32)
    out = _run(gpu_lib, H, We, ids, w, 8).cpu().numpy()
    assert np.all(np.isnan(out[[3, 7]]))
    ok = [t for t in range(T) if t not in (3, 7)]
    assert np.all(np.isfinite(out[ok]))
