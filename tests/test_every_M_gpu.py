"""GPU: every batch size gives every row the same bits.

[BitRL, section 2 and 4.1]: one accumulation order for every M, so a row's
result may not depend on how many rows share its call.  The linear layer
(4096 x 4096, 8 leaves) is called with every M from 1 to 4097 rows, each
result compared bit for bit with the first M rows of the 4097-row call; the
calls cover every tile height the schedule picks (64, 128 and 192 rows), every
ragged last m-tile and grids from one workgroup to several tiles per
workgroup.  The fused logprob is swept the same way over M = 1 .. 600 on
smaller LM heads: K = 1024, V = 5000 at 8 and at 16 leaves (64-column leaves),
K = 2048, V = 5000 at 16 leaves, and the full 151936-token vocabulary at
K = 512, 8 leaves.  Up to 192 rows a call has a single row of tiles (the sampled
logit picked inside the tile kernel); above, 128- and 192-row tiles alternate
as M grows, and at 16 leaves the 192-row tiles park the first half of the leaf
tree outside registers.  The 16-leaf contraction (K = 2048, N = 1024) is swept
over every M from 1 to 1024 (64- and 128-row tiles).  The block-FP8 path
(per-token quantisation of the first M rows, then the W8A8 contraction, FP32
and bf16 outputs), the MoE contraction + combine and the router (logits,
chosen experts, gates) are swept over every batch size up to 600 or 300 rows,
and the expert GEMMs over every row count 1 .. 400 of one expert, in both
layouts.  Comparisons run on the device.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu


def _first_mismatch(a: torch.Tensor, b: torch.Tensor):
    ne = (a.view(torch.int32) != b.view(torch.int32))
    if not bool(ne.any()):
        return None
    return tuple(int(i) for i in ne.nonzero()[0])


def test_linear_every_M_1_to_4097(gpu_lib):
    cfg = wl.CONFIGS["linear"]
    s = wl.streams(cfg.seed)
    Mmax = 4097
    A = dev_bf16(wl.normal_bf16(s["H"], (Mmax, cfg.K), 1.0))
    W = dev_bf16(wl.normal_bf16(s["W"], (cfg.N, cfg.K), 0.02))
    full = torch.empty(Mmax, cfg.N, dtype=torch.float32, device="cuda:0")
    gpu_lib.tig_tree_gemm(A, W, full, cfg.leaves)
    out = torch.empty_like(full)
    bad = []
    for M in range(1, Mmax + 1):
        if M % 512 == 1:
            say(f"linear every M: M = {M} ..")
        C = out[:M]
        gpu_lib.tig_tree_gemm(A[:M], W, C, cfg.leaves)
        where = _first_mismatch(C, full[:M])
        if where is not None:
            bad.append((M, where))
            if len(bad) >= 5:
                break
    torch.cuda.synchronize()
    assert not bad, f"rows differ from the 4097-row call at (M, (row, col)): {bad}"


@pytest.mark.parametrize("K,V,L", [(1024, 5000, 8), (1024, 5000, 16), (2048, 5000, 16), (512, 151936, 8)])
def test_logprob_every_M_1_to_600(gpu_lib, K, V, L):
    Mmax = 600
    rng = np.random.default_rng(20241 + K + V + L)
    H = dev_bf16(wl.normal_bf16(rng, (Mmax, K), 1.0))
    W = dev_bf16(wl.normal_bf16(rng, (V, K), 0.03))
    ids = torch.from_numpy(rng.integers(0, V, size=Mmax)).to("cuda:0")
    ws = torch.empty(gpu_lib.tig_logprob_workspace_bytes(Mmax, K, V, L), dtype=torch.uint8, device="cuda:0")
    full_lp = torch.empty(Mmax, dtype=torch.float32, device="cuda:0")
    full_lse = torch.empty_like(full_lp)
    gpu_lib.tig_logprob_gather(H, W, ids, full_lp, full_lse, L, ws)
    lp = torch.empty_like(full_lp)
    lse = torch.empty_like(full_lp)
    bad = []
    for M in range(1, Mmax + 1):
        if M % 100 == 1:
            say(f"logprob every M (K={K} V={V} L={L}): M = {M} ..")
        gpu_lib.tig_logprob_gather(H[:M], W, ids[:M], lp[:M], lse[:M], L, ws)
        for name, got, ref in (("logprob", lp[:M], full_lp[:M]), ("lse", lse[:M], full_lse[:M])):
            where = _first_mismatch(got, ref)
            if where is not None:
                bad.append((name, M, where))
        if len(bad) >= 5:
            break
    torch.cuda.synchronize()
    assert bool(torch.isfinite(full_lp).all())
    assert not bad, f"rows differ from the 600-row call: {bad}"


def test_tree_gemm_16_leaves_every_M_1_to_1024(gpu_lib):
    K, N, L, Mmax = 2048, 1024, 16, 1024
    rng = np.random.default_rng(77)
    A = dev_bf16(wl.normal_bf16(rng, (Mmax, K), 1.0))
    W = dev_bf16(wl.normal_bf16(rng, (N, K), 0.02))
    full = torch.empty(Mmax, N, dtype=torch.float32, device="cuda:0")
    gpu_lib.tig_tree_gemm(A, W, full, L)
    out = torch.empty_like(full)
    bad = []
    for M in range(1, Mmax + 1):
        if M % 256 == 1:
            say(f"16-leaf contraction every M: M = {M} ..")
        C = out[:M]
        gpu_lib.tig_tree_gemm(A[:M], W, C, L)
        where = _first_mismatch(C, full[:M])
        if where is not None:
            bad.append((M, where))
            if len(bad) >= 5:
                break
    torch.cuda.synchronize()
    assert not bad, f"rows differ from the 1024-row call at (M, (row, col)): {bad}"


@pytest.mark.parametrize("K,N,L,bf16", [(2048, 640, 8, False), (2048, 400, 16, True)])
def test_fp8_every_M_1_to_600(gpu_lib, K, N, L, bf16):
    """Quantise + W8A8 contraction of the first M rows, every M: the per-token
    activation blocks and the per-call scale table (sized by M) may not change
    a row's bits."""
    Mmax = 600
    rng = np.random.default_rng(31000 + N + L)
    A = dev_bf16(wl.normal_bf16(rng, (Mmax, K), 1.0))
    QW, SW = gpu_lib.fp8_quantize(dev_bf16(wl.normal_bf16(rng, (N, K), 0.02)), 128)
    dt = torch.bfloat16 if bf16 else torch.float32
    QA, SA = gpu_lib.fp8_quantize(A, 1)
    full = gpu_lib.fp8_tree_gemm(QA, SA, QW, SW, L, out_dtype=dt)
    view = torch.int16 if bf16 else torch.int32
    bad = []
    for M in range(1, Mmax + 1):
        if M % 100 == 1:
            say(f"fp8 every M (K={K} N={N} L={L} bf16={bf16}): M = {M} ..")
        qa, sa = gpu_lib.fp8_quantize(A[:M], 1)
        C = gpu_lib.fp8_tree_gemm(qa, sa, QW, SW, L, out_dtype=dt)
        ne = C.view(view) != full[:M].view(view)
        if bool(ne.any()):
            bad.append((M, tuple(int(i) for i in ne.nonzero()[0])))
            if len(bad) >= 5:
                break
    torch.cuda.synchronize()
    assert not bad, f"rows differ from the 600-row call at (M, (row, col)): {bad}"


@pytest.mark.parametrize("L", [8, 16])
def test_moe_every_T_1_to_300(gpu_lib, L):
    """The MoE contraction + combine of the first T tokens, every T: a token's
    output may not depend on how many tokens (and so how many rows per expert)
    share the call."""
    T, E, N, K, topk = 300, 16, 384, 1024, 4
    rng = np.random.default_rng(32000 + L)
    H = dev_bf16(wl.normal_bf16(rng, (T, K), 1.0))
    We = dev_bf16(wl.normal_bf16(rng, (E, N, K), 0.02))
    ids, w = wl.routing_input(rng, T, E, topk)
    ids, w = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    full = gpu_lib.moe_tree_gemm_combine(H, We, ids, w, L)
    ws = torch.empty(gpu_lib.tig_moe_workspace_bytes(T, N, K, E, topk), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(full)
    bad = []
    for t in range(1, T + 1):
        if t % 50 == 1:
            say(f"moe every T ({L} leaves): T = {t} ..")
        gpu_lib.tig_moe_tree_gemm_combine(H[:t], We, ids[:t], w[:t], out[:t], L, ws)
        where = _first_mismatch(out[:t], full[:t])
        if where is not None:
            bad.append((t, where))
            if len(bad) >= 5:
                break
    torch.cuda.synchronize()
    assert not bad, f"tokens differ from the 300-token call at (T, (token, col)): {bad}"


@pytest.mark.parametrize("E,topk,L", [(64, 8, 8), (100, 6, 8), (64, 8, 16)])
def test_router_every_T_1_to_300(gpu_lib, E, topk, L):
    """Router logits, chosen experts and gates of the first T tokens, every T."""
    T, K = 300, 2048
    rng = np.random.default_rng(33000 + E + L)
    H = dev_bf16(wl.normal_bf16(rng, (T, K), 1.0))
    Wr = dev_bf16(wl.normal_bf16(rng, (E, K), 0.02))
    f_lg, f_ids, f_w = gpu_lib.moe_route(H, Wr, topk, L)
    bad = []
    for t in range(1, T + 1):
        if t % 50 == 1:
            say(f"router every T (E={E} top-{topk}, {L} leaves): T = {t} ..")
        lg, ids, w = gpu_lib.moe_route(H[:t], Wr, topk, L)
        for name, got, ref in (("logits", lg.view(torch.int32), f_lg[:t].view(torch.int32)),
                               ("ids", ids, f_ids[:t]), ("gates", w.view(torch.int32), f_w[:t].view(torch.int32))):
            ne = got != ref
            if bool(ne.any()):
                bad.append((name, t, tuple(int(i) for i in ne.nonzero()[0])))
        if len(bad) >= 5:
            break
    torch.cuda.synchronize()
    assert not bad, f"tokens differ from the 300-token call: {bad}"


@pytest.mark.parametrize("L", [8, 16])
def test_expert_gemm_every_count_1_to_400(gpu_lib, L):
    """Expert GEMMs with expert 1 holding c rows, every c: its rows keep their bits
    as c grows (one tile row, several, ragged last tiles), in the masked layout and
    in the contiguous one (where expert 2's block moves with c), and experts 0 and
    2 are unchanged."""
    E, K, N, cap, align = 3, 1024, 320, 400, 128
    rng = np.random.default_rng(34000 + L)
    X = dev_bf16(wl.normal_bf16(rng, (E, cap, K), 1.0))
    W = dev_bf16(wl.normal_bf16(rng, (E, N, K), 0.02))
    fixed = (37, 150)
    full = gpu_lib.expert_gemm_masked(X, torch.tensor([fixed[0], cap, fixed[1]], dtype=torch.int32,
                                                       device="cuda:0"), W, L)
    up = lambda n: -(-n // align) * align
    bad = []
    for c in range(1, cap + 1):
        if c % 100 == 1:
            say(f"expert gemm every count ({L} leaves): c = {c} ..")
        counts = torch.tensor([fixed[0], c, fixed[1]], dtype=torch.int32, device="cuda:0")
        Ym = gpu_lib.expert_gemm_masked(X, counts, W, L)
        s1 = up(fixed[0])
        s2 = s1 + up(c)
        Xc = torch.zeros(s2 + fixed[1] + 5, K, dtype=torch.bfloat16, device="cuda:0")
        Xc[:fixed[0]] = X[0, :fixed[0]]
        Xc[s1:s1 + c] = X[1, :c]
        Xc[s2:s2 + fixed[1]] = X[2, :fixed[1]]
        Yc = gpu_lib.expert_gemm_contiguous(Xc, counts, W, align, L)
        pieces = (("masked expert 1", Ym[1, :c], full[1, :c]),
                  ("masked expert 0", Ym[0, :fixed[0]], full[0, :fixed[0]]),
                  ("masked expert 2", Ym[2, :fixed[1]], full[2, :fixed[1]]),
                  ("contiguous expert 1", Yc[s1:s1 + c], full[1, :c]),
                  ("contiguous expert 2", Yc[s2:s2 + fixed[1]], full[2, :fixed[1]]))
        for name, got, ref in pieces:
            where = _first_mismatch(got, ref)
            if where is not None:
                bad.append((name, c, where))
        if len(bad) >= 5:
            break
    torch.cuda.synchronize()
    assert not bad, f"rows differ from the full-count call: {bad}"
