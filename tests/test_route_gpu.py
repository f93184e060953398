"""GPU parity and batch invariance of tig_moe_route (the MoE router on the GPU).

[BitRL, section 4.1]: the router gate is one GEMM with FP32 output at every
batch size, so recomputed routing matches; [BitRL, section 1]: once the logits
match, the top-k tie-breaking and output order must be fixed as well.  Reading
used here: largest logit first, equal logits in ascending expert id; gates =
softmax over the selected logits.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bitwise, assert_gemm_close, dev_bf16, say

pytestmark = pytest.mark.gpu

GATE_ATOL = 2e-6   # hardware exp2 (about 1 ulp), a tree of <= 16 sums and one division


def _route(gpu_lib, H, Wr, topk, L):
    return gpu_lib.moe_route(dev_bf16(H), dev_bf16(Wr), topk, L)


def _valid_order(logits, ids):
    """Selected logits (the kernel's own) come first, descending, ties by lower id."""
    for t in range(logits.shape[0]):
        row = logits[t]
        sel = ids[t].tolist()
        assert len(set(sel)) == len(sel)
        for a, b in zip(sel, sel[1:]):
            assert row[a] > row[b] or (row[a] == row[b] and a < b), (t, a, b)
        rest = np.setdiff1d(np.arange(row.size), sel)
        if rest.size:
            worst = sel[-1]
            assert np.all((row[rest] < row[worst]) | ((row[rest] == row[worst]) & (rest > worst))), t


@pytest.mark.parametrize("E,topk", [(16, 1), (16, 3), (64, 8), (100, 8), (1024, 16)])
def test_route_integer_exact(gpu_lib, E, topk):
    """Small integers: the logits are exact (many ties), so ids match the oracle bit for bit."""
    rng = np.random.default_rng(900 + E + topk)
    T, K = 333, 512
    H = wl.integer_bf16(rng, (T, K), -2, 2)
    Wr = wl.integer_bf16(rng, (E, K), -1, 1)
    say(f"route integer E={E} topk={topk}")
    logits, ids, w = _route(gpu_lib, H, Wr, topk, 8)
    exact = oracle.contraction_ref(H, Wr)
    assert np.array_equal(logits.cpu().numpy().astype(np.float64), exact)
    ref_ids = oracle.route_select(exact, topk)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ref_w = oracle.route_gates_ref(exact, ref_ids)
    assert np.max(np.abs(w.cpu().numpy() - ref_w)) <= GATE_ATOL
    assert any(len(set(r)) < E for r in exact.tolist())   # ties were present


def test_route_equal_logits_take_lowest_ids(gpu_lib):
    T, K, E = 7, 512, 64
    H = wl.f32_to_bf16_bits(np.ones((T, K), dtype=np.float32))
    Wr = wl.f32_to_bf16_bits(np.full((E, K), 0.25, dtype=np.float32))
    logits, ids, w = _route(gpu_lib, H, Wr, 8, 8)
    assert np.all(ids.cpu().numpy() == np.arange(8))
    assert np.all(w.cpu().numpy() == np.float32(1 / 8))


def test_route_moe_config_parity_and_order(gpu_lib):
    """Router of the MoE config: 4096 tokens, hidden 2048, 64 experts, top-8, 8 leaves."""
    cfg = wl.CONFIGS["moe"]
    s = wl.streams(cfg.seed)
    H = wl.normal_bf16(s["H"], (cfg.tokens, cfg.K), 1.0)
    Wr = wl.normal_bf16(s["router"], (cfg.experts, cfg.K), 0.02)
    say("route parity: 4096 tokens, 64 experts, top-8")
    logits, ids, w = _route(gpu_lib, H, Wr, cfg.topk, cfg.leaves)
    lg, ids_np, w_np = logits.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    ref_logits, ref_ids, ref_w = oracle.route_ref(H, Wr, cfg.topk)
    assert_gemm_close(lg, ref_logits, what="router logits")
    _valid_order(lg, ids_np)
    # The selection is an integer decision on FP32 logits: taken by the oracle's
    # rule on the kernel's own FP32 logits (exact in fp64), it is the kernel's,
    # on every row; so are the gates, within the exp2 / division tolerance.
    lg64 = lg.astype(np.float64)
    assert np.array_equal(ids_np, oracle.route_select(lg64, cfg.topk))
    assert np.max(np.abs(w_np - oracle.route_gates_ref(lg64, ids_np))) <= GATE_ATOL
    # Where the oracle's ranking has a clear margin, the selection is the oracle's.
    srt = -np.sort(-ref_logits, axis=1)
    gaps = np.abs(np.diff(srt[:, :cfg.topk + 1], axis=1)).min(axis=1)
    clear = gaps > 1e-3
    assert clear.mean() > 0.5
    assert np.array_equal(ids_np[clear], ref_ids[clear])
    assert np.max(np.abs(w_np[clear] - ref_w[clear])) <= 1e-5
    assert np.allclose(w_np.sum(axis=1), 1.0, atol=1e-6)


def test_route_batch_invariance(gpu_lib):
    """4096 tokens at once, in 32 batches of 128, and single tokens: the same bits."""
    cfg = wl.CONFIGS["moe"]
    s = wl.streams(cfg.seed)
    H = dev_bf16(wl.normal_bf16(s["H"], (cfg.tokens, cfg.K), 1.0))
    Wr = dev_bf16(wl.normal_bf16(s["router"], (cfg.experts, cfg.K), 0.02))
    full = gpu_lib.moe_route(H, Wr, cfg.topk, cfg.leaves)
    parts = [gpu_lib.moe_route(H[i:i + 128].contiguous(), Wr, cfg.topk, cfg.leaves) for i in range(0, 4096, 128)]
    for k, name in enumerate(("logits", "ids", "gates")):
        assert_bitwise(torch.cat([p[k] for p in parts]), full[k], f"route {name}, 32 x 128 vs 4096")
    for r in (0, 1, 777, 4095):
        one = gpu_lib.moe_route(H[r:r + 1].contiguous(), Wr, cfg.topk, cfg.leaves)
        for k, name in enumerate(("logits", "ids", "gates")):
            assert_bitwise(one[k], full[k][r:r + 1], f"route {name}, token {r} alone")


def test_routed_moe_is_batch_invariant(gpu_lib):
    """GPU router, then the MoE contraction and combine: the same bits for any batch split."""
    rng = np.random.default_rng(905)
    T, K, N, E, topk = 512, 512, 256, 16, 4
    H = dev_bf16(wl.normal_bf16(rng, (T, K), 1.0))
    Wr = dev_bf16(wl.normal_bf16(rng, (E, K), 0.05))
    We = dev_bf16(wl.normal_bf16(rng, (E, N, K), 0.05))

    def run(h):
        _, ids, w = gpu_lib.moe_route(h, Wr, topk, 8)
        return gpu_lib.moe_tree_gemm_combine(h, We, ids, w, 8)

    full = run(H)
    parts = torch.cat([run(H[i:i + 64].contiguous()) for i in range(0, T, 64)])
    assert_bitwise(parts, full, "router + MoE, 8 x 64 vs 512 tokens")


@pytest.mark.parametrize("T,E,K,L", [(333, 16, 512, 1), (4096, 64, 2048, 8), (1000, 100, 1024, 2),
                                     (77, 1024, 2048, 16), (4096, 64, 2048, 4), (50, 64, 4096, 8),
                                     (129, 130, 768, 4)])
def test_route_logits_equal_tree_gemm(gpu_lib, T, E, K, L):
    """The router's logits are the leaf-tree contraction with FP32 output: bit for bit
    what tig_tree_gemm gives for the same H and Wr (ragged T and E, 1 .. 16 leaves)."""
    rng = np.random.default_rng(4242 + T + E + K + L)
    H = dev_bf16(wl.normal_bf16(rng, (T, K), 1.0))
    Wr = dev_bf16(wl.normal_bf16(rng, (E, K), 0.02))
    logits, _, _ = gpu_lib.moe_route(H, Wr, min(8, E), L)
    C = torch.empty(T, E, dtype=torch.float32, device="cuda:0")
    gpu_lib.tig_tree_gemm(H, Wr, C, L)
    assert_bitwise(logits, C, f"router logits vs tree GEMM T={T} E={E} K={K} L={L}")
