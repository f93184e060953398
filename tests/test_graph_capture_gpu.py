"""GPU: every entry point inside one captured graph, replayed.

The library clears its workspaces with kernels of its own (it issues no
memset, allocation or copy), so a serving loop can capture a whole step in a
HIP graph with workspaces allocated beforehand.  One graph holds a step of
every path: the router and the MoE contraction + combine it feeds, an
expert GEMM and SiLU * up, the tree GEMM, the fused logprob, block-FP8
quantisation and the W8A8 GEMM, and the Top-K.  It is replayed four times;
between replays the outputs are overwritten, the same entry points run
eagerly on other inputs, and the host synchronises.  Every replay must give
the eager results bit for bit ([BitRL, section 4.6]: no host round trips,
workspaces sized from static bounds).
"""

import numpy as np
import torch
import pytest

import workloads as wl
from gpu_util import assert_bitwise, dev_bf16, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else (
        t.view(torch.int32) if t.dtype == torch.float32 else t)


def test_one_graph_of_every_entry_point_replays_bitwise(gpu_lib):
    rng = np.random.default_rng(36000)
    L = 8
    # MoE: router -> combine
    T, E, K, N, topk = 512, 16, 1024, 384, 4
    H = dev_bf16(wl.normal_bf16(rng, (T, K), 1.0))
    Wr = dev_bf16(wl.normal_bf16(rng, (E, K), 0.02))
    We = dev_bf16(wl.normal_bf16(rng, (E, N, K), 0.02))
    logits = torch.empty(T, E, device=DEV)
    rid = torch.empty(T, topk, dtype=torch.int32, device=DEV)
    rw = torch.empty(T, topk, device=DEV)
    moe_out = torch.empty(T, N, device=DEV)
    ws_moe = torch.empty(gpu_lib.tig_moe_workspace_bytes(T, N, K, E, topk), dtype=torch.uint8, device=DEV)
    # expert GEMM (masked) and SiLU * up
    cap = 192
    Xm = dev_bf16(wl.normal_bf16(rng, (E, cap, K), 1.0))
    W13 = dev_bf16(wl.normal_bf16(rng, (E, 2 * 256, K), 0.02))
    counts = torch.from_numpy(rng.integers(0, cap + 1, size=E).astype(np.int32)).to(DEV)
    G = torch.empty(E, cap, 2 * 256, device=DEV)
    ws_e = torch.empty(max(gpu_lib.tig_expert_workspace_bytes(E * cap, E), 256), dtype=torch.uint8, device=DEV)
    act = torch.empty(E * cap, 256, dtype=torch.bfloat16, device=DEV)
    # tree GEMM and fused logprob
    M, V = 300, 5000
    A = dev_bf16(wl.normal_bf16(rng, (M, K), 1.0))
    Wv = dev_bf16(wl.normal_bf16(rng, (V, K), 0.03))
    C = torch.empty(M, V, device=DEV)
    ids = torch.from_numpy(rng.integers(0, V, size=M)).to(DEV)
    lp = torch.empty(M, device=DEV)
    lse = torch.empty(M, device=DEV)
    ws_lp = torch.empty(gpu_lib.tig_logprob_workspace_bytes(M, K, V, L), dtype=torch.uint8, device=DEV)
    # block FP8
    QW, SW = gpu_lib.fp8_quantize(Wv[:640], 128)
    QA = torch.empty(M, K, dtype=torch.uint8, device=DEV)
    SA = torch.empty(M, K // 128, dtype=torch.uint8, device=DEV)
    C8 = torch.empty(M, 640, device=DEV)
    ws8 = torch.empty(max(gpu_lib.tig_fp8_gemm_workspace_bytes(M, 640, K), 256), dtype=torch.uint8, device=DEV)
    # Top-K
    R, ld, k = 32, 8192, 512
    scores = torch.from_numpy(wl.indexer_scores(rng, R, ld, "bf16")).to(DEV)
    lengths = torch.from_numpy(wl.request_lengths(rng, R, 1, ld)).to(DEV)
    tk = torch.empty(R, k, dtype=torch.int32, device=DEV)

    def step():
        gpu_lib.tig_moe_route(H, Wr, logits, rid, rw, L)
        gpu_lib.tig_moe_tree_gemm_combine(H, We, rid, rw, moe_out, L, ws_moe)
        gpu_lib.tig_expert_gemm_masked(Xm, counts, W13, G, L, ws_e)
        gpu_lib.tig_silu_mul(G.view(E * cap, 2 * 256), act)
        gpu_lib.tig_tree_gemm(A, Wv, C, L)
        gpu_lib.tig_logprob_gather(A, Wv, ids, lp, lse, L, ws_lp)
        gpu_lib.tig_fp8_quantize(A, QA, SA, 1)
        gpu_lib.tig_fp8_tree_gemm(QA, SA, QW, SW, C8, L, ws8)
        gpu_lib.tig_topk_positions(scores, lengths, tk)

    outs = {"logits": logits, "ids": rid, "gates": rw, "moe": moe_out, "expert": G, "silu": act, "gemm": C,
            "logprob": lp, "lse": lse, "qa": QA, "sa": SA, "fp8 gemm": C8, "topk": tk}
    say("graph: eager step")
    step()
    torch.cuda.synchronize()
    ref = {name: t.clone() for name, t in outs.items()}
    # Rows whose expert count is 0 are not written: compare only the counted rows.
    cnt = counts.cpu().numpy()

    def check(tag):
        for name, t in outs.items():
            if name in ("expert", "silu"):
                tv = t.view(E, cap, -1)
                rv = ref[name].view(E, cap, -1)
                for e in range(E):
                    c = int(cnt[e])
                    if c:
                        assert_bitwise(tv[e, :c], rv[e, :c], f"{tag} {name} expert {e}")
            else:
                assert torch.equal(_bits(t), _bits(ref[name])), f"{tag}: {name} differs"

    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                      # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    # eager work on other inputs between the replays
    H2 = dev_bf16(wl.normal_bf16(rng, (T, K), 1.0))
    A2 = dev_bf16(wl.normal_bf16(rng, (M, K), 1.0))
    for rep in range(4):
        say(f"graph replay {rep}")
        for t in outs.values():
            t.fill_(7 if t.dtype in (torch.int32, torch.uint8) else -3.0)
        o1 = torch.empty(T, E, device=DEV)
        gpu_lib.tig_moe_route(H2, Wr, o1, torch.empty_like(rid), torch.empty_like(rw), L)
        gpu_lib.tig_logprob_gather(A2, Wv, ids, torch.empty_like(lp), None, L, ws_lp)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        check(f"replay {rep}")
