"""GPU: decode-sized logprob calls (one row of tiles) against batch rows.

A batch of at most 192 rows runs as a single row of tiles (128 rows up to
128, 192 rows above): each W tile is read by one workgroup only (non-temporal
loads) and the workgroups of an XCD start at staggered leaves; a batch of
more rows shares each W tile among its row tiles.  [BitRL, section 2]: a token's logprob must not depend
on the batch it arrives in, so each row of a decode-sized call must equal,
bit for bit, the same row computed inside a batch of 200 rows, for logprob
and lse, at ragged vocabularies (a last tile with 1, 104 or 11 of its 128
columns, or a vocabulary of one), rows past M in the tile, several leaf counts
and leaf lengths, and workgroups that run many tiles.  The fp64 oracle bounds
the values (|delta| <= 1e-3).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bitwise, dev_bf16, record, say

pytestmark = pytest.mark.gpu

BIG = 200   # rows of the reference batch: two 128-row tiles


@pytest.mark.parametrize("K,L", [(512, 1), (1024, 2), (2048, 4), (4096, 8), (8192, 8)])
@pytest.mark.parametrize("V", [1, 129, 1000, 5003])
def test_decode_rows_equal_batch_rows(gpu_lib, K, L, V):
    rng = np.random.default_rng(K * 7919 + L * 131 + V)
    H = wl.normal_bf16(rng, (BIG, K), 1.0)
    W = wl.normal_bf16(rng, (V, K), 0.03)
    ids = rng.integers(0, V, size=BIG)
    Hd, Wd, idd = dev_bf16(H), dev_bf16(W), torch.from_numpy(ids).cuda()
    say(f"decode vs batch K={K} L={L} V={V}: batch of {BIG}")
    ref_lp, ref_lse = gpu_lib.logprob_gather(Hd, Wd, idd, L)
    for a, b in [(0, 1), (5, 42), (0, 128), (72, 200)]:
        say(f"decode vs batch K={K} L={L} V={V}: rows [{a}, {b})")
        lp, lse = gpu_lib.logprob_gather(Hd[a:b].contiguous(), Wd, idd[a:b].contiguous(), L)
        assert_bitwise(lp, ref_lp[a:b], f"logprob rows [{a},{b}) K={K} L={L} V={V}")
        assert_bitwise(lse, ref_lse[a:b], f"lse rows [{a},{b}) K={K} L={L} V={V}")
    if K <= 2048:
        o_lp, o_lse = oracle.logprob_ref(H[:42], W, ids[:42])
        lp, lse = gpu_lib.logprob_gather(Hd[:42], Wd, idd[:42], L)
        e1 = float(np.max(np.abs(lp.cpu().double().numpy() - o_lp)))
        e2 = float(np.max(np.abs(lse.cpu().double().numpy() - o_lse)))
        say(f"  oracle: max |dlogprob| {e1:.2e}, max |dlse| {e2:.2e}")
        record("oracle_logprob", f"decode K={K} L={L} V={V} rows 0..41", rows=42, max_abs_logprob=e1,
               max_abs_lse=e2, bound=1e-3)
        assert e1 <= 1e-3 and e2 <= 1e-3


def test_decode_repeat_and_many_tiles_per_workgroup(gpu_lib):
    """2000 vocabulary tiles: every workgroup runs several tiles (alternating
    leaf order, epilogue region reused); repeated calls give the same bits."""
    K, L, V, M = 4096, 8, 256000, 96
    rng = np.random.default_rng(31337)
    H = dev_bf16(wl.normal_bf16(rng, (BIG, K), 1.0))
    W = dev_bf16(wl.normal_bf16(rng, (V, K), 0.02))
    ids = torch.from_numpy(rng.integers(0, V, size=BIG)).cuda()
    say(f"decode many tiles K={K} L={L} V={V} M={M}")
    ref_lp, ref_lse = gpu_lib.logprob_gather(H, W, ids, L)
    first = None
    for rep in range(3):
        lp, lse = gpu_lib.logprob_gather(H[:M].contiguous(), W, ids[:M].contiguous(), L)
        assert_bitwise(lp, ref_lp[:M], f"logprob many tiles, call {rep}")
        assert_bitwise(lse, ref_lse[:M], f"lse many tiles, call {rep}")
        if first is None:
            first = lp.clone()
        assert_bitwise(lp, first, f"repeat {rep}")
