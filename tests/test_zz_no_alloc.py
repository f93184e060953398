"""tig_logprob_gather_noalloc against tig_logprob_gather (GPU).

The no-allocation entry point runs the same kernels on the library's fixed
device array instead of a caller's workspace, so its outputs must be the same
bits.  Two calls in a row, the second on fewer rows, check that the array's
leftover contents from the first call do not leak into the second.  The
16-leaf case with more than 128 rows takes the split-tree path, whose parked
half trees also live in the array.  The call is also captured in a graph and
replayed, the use it exists for.
"""

import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import assert_bitwise, dev_bf16, say


def _inputs(seed, M, K, V):
    s = wl.streams(seed)
    H = wl.normal_bf16(s["H"], (M, K), 1.0)
    W = wl.normal_bf16(s["W"], (V, K), 0.02)
    ids = wl.uniform_ids(s["ids"], M, V)
    return dev_bf16(H), dev_bf16(W), torch.from_numpy(ids).to("cuda:0")


@pytest.mark.gpu
@pytest.mark.parametrize("K,V,leaves,M1,M2", [
    (1024, 5000, 8, 300, 37),      # several m-tiles, then one ragged tile
    (2048, 4097, 16, 150, 20),     # 16 leaves, 192-row tiles: the split tree's parked halves
    (1024, 151936, 8, 128, 1),     # decode-sized call at the LM-head vocabulary, then a single row
])
def test_noalloc_equals_workspace_entry_point(gpu_lib, K, V, leaves, M1, M2):
    tig = gpu_lib
    say(f"noalloc K={K} V={V} leaves={leaves} M={M1} then {M2}")
    H, W, ids = _inputs(4242 + leaves, M1, K, V)
    for M in (M1, M2):
        lp = torch.empty(M, dtype=torch.float32, device="cuda:0")
        lse = torch.empty(M, dtype=torch.float32, device="cuda:0")
        tig.tig_logprob_gather_noalloc(H[:M], W, ids[:M], lp, lse, leaves)
        ref_lp, ref_lse = tig.logprob_gather(H[:M], W, ids[:M], leaves)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(lp).all())
        assert_bitwise(lp, ref_lp, f"noalloc logprob M={M}")
        assert_bitwise(lse, ref_lse, f"noalloc lse M={M}")


@pytest.mark.gpu
def test_noalloc_rejects_calls_above_its_array(gpu_lib):
    tig = gpu_lib
    # 4000 rows x 1187 vocabulary tiles of partials: above the 32 MiB array
    lp = torch.empty(4000, dtype=torch.float32, device="cuda:0")
    big_H = torch.zeros((4000, 512), dtype=torch.bfloat16, device="cuda:0")
    big_W = torch.zeros((151936, 512), dtype=torch.bfloat16, device="cuda:0")
    big_ids = torch.zeros(4000, dtype=torch.int64, device="cuda:0")
    with pytest.raises(tig.TigError) as e:
        tig.tig_logprob_gather_noalloc(big_H, big_W, big_ids, lp, None, 8)
    assert e.value.status == tig.TIG_ERR_UNSUPPORTED


@pytest.mark.gpu
@pytest.mark.parametrize("K,V,leaves,M", [
    (1024, 5000, 8, 300),       # several m-tiles, the sampled logit by its own kernel
    (2048, 4097, 16, 150),      # 192-row tiles at 16 leaves: parked half trees in the array
    (1024, 151936, 8, 128),     # one row of tiles: the sampled logit inside the tile kernel
])
def test_noalloc_graph_replays_match_eager(gpu_lib, K, V, leaves, M):
    """The no-allocation call captured in a graph and replayed four times, with
    eager work between the replays (the buffers cleared, and an eager call on
    other rows that leaves its own data in the device array): every replay gives
    the eager call's bits."""
    tig = gpu_lib
    say(f"noalloc graph K={K} V={V} leaves={leaves} M={M}")
    H, W, ids = _inputs(5151 + leaves, 2 * M, K, V)
    Hm, idm = H[:M].contiguous(), ids[:M].contiguous()
    ref_lp = torch.empty(M, dtype=torch.float32, device="cuda:0")
    ref_lse = torch.empty_like(ref_lp)
    tig.tig_logprob_gather_noalloc(Hm, W, idm, ref_lp, ref_lse, leaves)   # first call on the device: eager
    torch.cuda.synchronize()
    lp = torch.empty_like(ref_lp)
    lse = torch.empty_like(ref_lp)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tig.tig_logprob_gather_noalloc(Hm, W, idm, lp, lse, leaves)
    other_lp = torch.empty(M, dtype=torch.float32, device="cuda:0")
    for rep in range(4):
        lp.fill_(float("nan"))
        lse.fill_(float("nan"))
        tig.tig_logprob_gather_noalloc(H[M:].contiguous(), W, ids[M:].contiguous(), other_lp, None, leaves)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_bitwise(lp, ref_lp, f"graph replay {rep} logprob")
        assert_bitwise(lse, ref_lse, f"graph replay {rep} lse")
