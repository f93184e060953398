"""GPU: calls on two streams at once give the bits they give alone.

The entry points keep no state between calls (each brings its own workspace),
so work queued on two streams (default priority) and running concurrently
must give every output bit for bit as the same calls on one stream do
([BitRL, section 2]: a row's result does not depend on what else runs).
"""

import numpy as np
import torch
import pytest

import workloads as wl
from gpu_util import dev_bf16, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_two_streams_concurrent_equal_one_stream(gpu_lib):
    rng = np.random.default_rng(37000)
    L, K, V, M = 8, 1024, 20000, 700
    A = dev_bf16(wl.normal_bf16(rng, (M, K), 1.0))
    W = dev_bf16(wl.normal_bf16(rng, (V, K), 0.03))
    ids = torch.from_numpy(rng.integers(0, V, size=M)).to(DEV)
    B = dev_bf16(wl.normal_bf16(rng, (M, K), 1.0))
    T, E, N, topk = 1024, 16, 512, 4
    Hm = dev_bf16(wl.normal_bf16(rng, (T, K), 1.0))
    Wr = dev_bf16(wl.normal_bf16(rng, (E, K), 0.02))
    We = dev_bf16(wl.normal_bf16(rng, (E, N, K), 0.02))

    ws1 = torch.empty(gpu_lib.tig_logprob_workspace_bytes(M, K, V, L), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty(gpu_lib.tig_moe_workspace_bytes(T, N, K, E, topk), dtype=torch.uint8, device=DEV)

    def outputs():
        return {"lp": torch.empty(M, device=DEV), "lse": torch.empty(M, device=DEV),
                "C": torch.empty(M, V, device=DEV), "lg": torch.empty(T, E, device=DEV),
                "rid": torch.empty(T, topk, dtype=torch.int32, device=DEV), "rw": torch.empty(T, topk, device=DEV),
                "moe": torch.empty(T, N, device=DEV)}

    def path1(o, s):
        gpu_lib.tig_logprob_gather(A, W, ids, o["lp"], o["lse"], L, ws1, stream=s)

    def path2(o, s):
        gpu_lib.tig_tree_gemm(B, W, o["C"], L, stream=s)
        gpu_lib.tig_moe_route(Hm, Wr, o["lg"], o["rid"], o["rw"], L, stream=s)
        gpu_lib.tig_moe_tree_gemm_combine(Hm, We, o["rid"], o["rw"], o["moe"], L, ws2, stream=s)

    ref = outputs()
    path1(ref, None)
    path2(ref, None)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        say(f"two streams, round {rep}")
        o = outputs()
        torch.cuda.synchronize()
        # both queues filled before either is waited on; the order of issue alternates
        if rep % 2 == 0:
            path1(o, s1)
            path2(o, s2)
        else:
            path2(o, s2)
            path1(o, s1)
        torch.cuda.synchronize()
        for name in ref:
            a, b = o[name], ref[name]
            va = a.view(torch.int32) if a.dtype == torch.float32 else a
            vb = b.view(torch.int32) if b.dtype == torch.float32 else b
            assert torch.equal(va, vb), f"round {rep}: {name} differs from the one-stream run"
