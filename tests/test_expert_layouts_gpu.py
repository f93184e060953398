"""GPU parity and layout invariance of the expert GEMMs and the activation.

[BitRL, section 4.4]: the rollout feeds the experts a masked layout (a
fixed-capacity block per expert), training a contiguous one (experts packed in
order with alignment padding); a row's expert result must be the same bits in
both, and the activation between the two expert GEMMs, SiLU(gate) * up, is
computed in FP32 and rounded to bf16 once.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_util import assert_bitwise, assert_gemm_close, dev_bf16, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _layouts(rng, rows_e, K, cap, align, extra=7):
    """The same expert rows in a masked [E, cap, K] and a contiguous [M, K]
    layout; every row no expert owns holds other values (bf16 of N(0, 25))."""
    E = len(rows_e)
    counts = np.array([r.shape[0] for r in rows_e], dtype=np.int32)
    Xm = wl.normal_bf16(rng, (E, cap, K), 5.0)
    for e, r in enumerate(rows_e):
        Xm[e, :min(r.shape[0], cap)] = r[:cap]
    starts, _ = oracle.expert_row_starts(counts, "contiguous", align=align)
    M = int(starts[-1] + counts[-1]) + extra
    Xc = wl.normal_bf16(rng, (M, K), 5.0)
    for e, r in enumerate(rows_e):
        Xc[starts[e]:starts[e] + r.shape[0]] = r
    return counts, Xm, Xc, starts


def _ws(gpu_lib, rows, E):
    return torch.empty(max(gpu_lib.tig_expert_workspace_bytes(rows, E), 256), dtype=torch.uint8, device=DEV)


def _masked(gpu_lib, Xm, counts, W, L, dtype=torch.float32):
    return gpu_lib.expert_gemm_masked(dev_bf16(Xm), torch.from_numpy(counts).to(DEV), dev_bf16(W), L, dtype)


def _contig(gpu_lib, Xc, counts, W, align, L, dtype=torch.float32):
    return gpu_lib.expert_gemm_contiguous(dev_bf16(Xc), torch.from_numpy(counts).to(DEV), dev_bf16(W), align, L,
                                          dtype)


EDGE_COUNTS = [0, 1, 127, 128, 129, 192, 193, 300, 5]


@pytest.mark.parametrize("align", [1, 128])
def test_expert_gemm_both_layouts_match_oracle_and_each_other(gpu_lib, align):
    rng = np.random.default_rng(3000 + align)
    E, K, N, L = len(EDGE_COUNTS), 512, 300, 8
    rows_e = [wl.normal_bf16(rng, (c, K), 1.0) for c in EDGE_COUNTS]
    W = wl.normal_bf16(rng, (E, N, K), 0.02)
    cap = 320
    counts, Xm, Xc, starts = _layouts(rng, rows_e, K, cap, align)
    say(f"expert gemm: E={E} K={K} N={N} cap={cap} align={align}")
    Ym = _masked(gpu_lib, Xm, counts, W, L).cpu().numpy()
    Yc = _contig(gpu_lib, Xc, counts, W, align, L).cpu().numpy()
    ref_m = oracle.expert_gemm_ref(Xm.reshape(E * cap, K), counts, W, "masked", cap=cap)
    ref_c = oracle.expert_gemm_ref(Xc, counts, W, "contiguous", align=align)
    for e, c in enumerate(EDGE_COUNTS):
        if c == 0:
            continue
        ym = Ym[e, :c]
        yc = Yc[starts[e]:starts[e] + c]
        assert_gemm_close(ym, ref_m[e * cap:e * cap + c], what=f"masked expert {e}")
        assert_gemm_close(yc, ref_c[starts[e]:starts[e] + c], what=f"contiguous expert {e}")
        assert np.array_equal(ym.view(np.uint32), yc.view(np.uint32)), f"layouts differ for expert {e}"


def test_expert_rows_equal_the_row_alone(gpu_lib):
    """A row's result equals tig_tree_gemm on that row alone against its expert's W."""
    rng = np.random.default_rng(3100)
    E, K, N, L = 4, 1024, 200, 16
    counts_l = [200, 3, 0, 64]
    rows_e = [wl.normal_bf16(rng, (c, K), 1.0) for c in counts_l]
    W = wl.normal_bf16(rng, (E, N, K), 0.02)
    counts, Xm, Xc, starts = _layouts(rng, rows_e, K, 256, 128)
    Ym = _masked(gpu_lib, Xm, counts, W, L)
    Yc = _contig(gpu_lib, Xc, counts, W, 128, L)
    Wd = dev_bf16(W)
    for e, c in enumerate(counts_l):
        for i in sorted({0, c // 2, c - 1}):
            if c == 0:
                continue
            alone = gpu_lib.tree_gemm(dev_bf16(rows_e[e][i:i + 1]), Wd[e], L)
            assert_bitwise(Ym[e, i:i + 1], alone, f"masked row {i} of expert {e}")
            assert_bitwise(Yc[starts[e] + i:starts[e] + i + 1], alone, f"contiguous row {i} of expert {e}")


def test_expert_gemm_bf16_output_is_the_rounded_f32(gpu_lib):
    rng = np.random.default_rng(3200)
    E, K, N, L = 3, 512, 256, 8
    rows_e = [wl.normal_bf16(rng, (c, K), 1.0) for c in (130, 0, 64)]
    W = wl.normal_bf16(rng, (E, N, K), 0.02)
    counts, Xm, Xc, starts = _layouts(rng, rows_e, K, 192, 1)
    f32 = _contig(gpu_lib, Xc, counts, W, 1, L).cpu().numpy()
    b16 = _contig(gpu_lib, Xc, counts, W, 1, L, torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
    for e, c in enumerate((130, 0, 64)):
        sl = slice(int(starts[e]), int(starts[e]) + c)
        assert np.array_equal(b16[sl], wl.f32_to_bf16_bits(f32[sl]))


def test_expert_gemm_repeat_calls_identical(gpu_lib):
    rng = np.random.default_rng(3250)
    E, K, N, L = 5, 1024, 384, 8
    counts_l = (300, 7, 0, 129, 64)
    rows_e = [wl.normal_bf16(rng, (c, K), 1.0) for c in counts_l]
    W = wl.normal_bf16(rng, (E, N, K), 0.02)
    counts, Xm, Xc, starts = _layouts(rng, rows_e, K, 320, 128)
    first = _masked(gpu_lib, Xm, counts, W, L)
    for _ in range(3):
        again = _masked(gpu_lib, Xm, counts, W, L)
        for e, c in enumerate(counts_l):          # rows no expert owns are not written
            assert_bitwise(again[e, :c], first[e, :c], f"masked repeat, expert {e}")


def test_expert_counts_clamped(gpu_lib):
    """Masked: a count above cap keeps the block's cap rows; below 0 counts as
    0.  Contiguous: rows that would lie past M are not computed (not written)."""
    rng = np.random.default_rng(3300)
    E, K, N, L, cap = 3, 512, 128, 8, 100
    W = wl.normal_bf16(rng, (E, N, K), 0.02)
    Xm = wl.normal_bf16(rng, (E, cap, K), 1.0)
    counts = np.array([150, -4, 100], dtype=np.int32)
    Ym = _masked(gpu_lib, Xm, counts, W, L).cpu().numpy()
    ref = oracle.expert_gemm_ref(Xm.reshape(E * cap, K), counts, W, "masked", cap=cap).reshape(E, cap, N)
    assert_gemm_close(Ym[0], ref[0], what="count above cap")
    assert_gemm_close(Ym[2], ref[2], what="count equal to cap")
    M = 120
    Xc = wl.normal_bf16(rng, (M, K), 1.0)
    counts_c = np.array([70, 80, 5], dtype=np.int32)        # segments 0..69, 70..149 (past M), 150..
    Yd = torch.full((M, N), 7.0, device=DEV)
    gpu_lib.tig_expert_gemm_contiguous(dev_bf16(Xc), torch.from_numpy(counts_c).to(DEV), dev_bf16(W), Yd, 1, L,
                                       _ws(gpu_lib, M, E))
    Yc = Yd.cpu().numpy()
    ref_c = oracle.contraction_ref(Xc, W[0])
    assert_gemm_close(Yc[:70], ref_c[:70], what="first segment")
    ref_1 = oracle.contraction_ref(Xc[70:], W[1])
    assert_gemm_close(Yc[70:], ref_1, what="second segment, cut at M")


def _near_midpoint(v, a_bits, b_bits, rel=2.0 ** -18):
    va, vb = oracle.bf16_bits_to_f64(a_bits), oracle.bf16_bits_to_f64(b_bits)
    return np.abs(v - (va + vb) / 2) <= rel * np.abs(v)


def test_silu_mul_matches_one_rounding(gpu_lib):
    """bf16(SiLU(g) u) equals the oracle's single rounding of the exact value,
    except within 2^-18 (relative) of a rounding midpoint, where FP32
    arithmetic cannot decide; there it is the neighbouring step."""
    rng = np.random.default_rng(3400)
    rows, I = 300, 1000
    GU = (rng.standard_normal((rows, 2 * I)) * 3).astype(np.float32)
    GU[0, :8] = [0.0, -0.0, 100.0, -100.0, 1e4, -1e4, 1e-30, -95.0]
    GU[0, I:I + 8] = [5.0, -5.0, 1.0, 1.0, 2.0, 3.0, 1.0, 1.0]
    say(f"silu_mul rows={rows} I={I}")
    got = gpu_lib.silu_mul(torch.from_numpy(GU).to(DEV)).cpu().view(torch.int16).numpy().view(np.uint16)
    g, u = GU[:, :I].astype(np.float64), GU[:, I:].astype(np.float64)
    ref = oracle.silu_mul_ref(g, u)
    with np.errstate(over="ignore"):
        v = g / (1.0 + np.exp(-g)) * u
    # Below FP32's normal range the result depends on whether the hardware exp2
    # keeps denormals: there it is the oracle's value or a zero of its sign.
    tiny = np.abs(v) < 2.0 ** -126
    assert np.all((got[tiny] == ref[tiny]) | (got[tiny] & 0x7FFF == 0) & ((got[tiny] ^ ref[tiny]) & 0x8000 == 0))
    diff = (got != ref) & ~tiny
    assert np.all(_near_midpoint(v[diff], got[diff], ref[diff])), int(diff.sum())
    assert np.all(np.abs(got[diff].astype(np.int32) - ref[diff].astype(np.int32)) == 1)
    assert diff.sum() <= 0.001 * diff.size
    assert got[0, :7].tolist() == ref[0, :7].tolist()
    # rounding SiLU first would change many of these results: not what is computed
    with np.errstate(over="ignore"):
        twice = oracle.f64_to_bf16_rne(oracle.bf16_bits_to_f64(oracle.f64_to_bf16_rne(g / (1.0 + np.exp(-g)))) * u)
    split = (twice != ref) & ~_near_midpoint(v, ref, twice) & ~tiny
    assert split.sum() > 100
    assert np.array_equal(got[split], ref[split])


def test_silu_mul_strided_and_odd_widths(gpu_lib):
    rng = np.random.default_rng(3500)
    GU = torch.from_numpy((rng.standard_normal((17, 2 * 37 + 5)) * 2).astype(np.float32)).to(DEV)
    view = GU[:, :74]                                         # row stride 79, I = 37 (scalar path)
    out = torch.empty(17, 37, dtype=torch.bfloat16, device=DEV)
    gpu_lib.tig_silu_mul(view, out)
    g = view[:, :37].cpu().numpy().astype(np.float64)
    u = view[:, 37:].cpu().numpy().astype(np.float64)
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.silu_mul_ref(g, u)
    diff = got != ref
    assert np.all(_near_midpoint((g / (1.0 + np.exp(-g)) * u)[diff], got[diff], ref[diff]))


def test_expert_ffn_same_bits_on_both_layouts(gpu_lib):
    """gate/up GEMM, SiLU * up, down GEMM: every row the same bits in the masked
    and the contiguous layout, and close to the fp64 chain with one rounding
    of the activation."""
    rng = np.random.default_rng(3600)
    E, H, I, L = 6, 512, 512, 8
    counts_l = [40, 0, 200, 1, 129, 64]
    rows_e = [wl.normal_bf16(rng, (c, H), 1.0) for c in counts_l]
    W13 = wl.normal_bf16(rng, (E, 2 * I, H), 0.05)
    W2 = wl.normal_bf16(rng, (E, H, I), 0.05)
    counts, Xm, Xc, starts = _layouts(rng, rows_e, H, 256, 128)
    cd = torch.from_numpy(counts).to(DEV)
    W13d, W2d = dev_bf16(W13), dev_bf16(W2)
    say("expert ffn: masked")
    G = gpu_lib.expert_gemm_masked(dev_bf16(Xm), cd, W13d, L)
    Am = gpu_lib.silu_mul(G.reshape(E * 256, 2 * I)).reshape(E, 256, I)
    Ym = gpu_lib.expert_gemm_masked(Am, cd, W2d, L).cpu().numpy()
    say("expert ffn: contiguous")
    Gc = gpu_lib.expert_gemm_contiguous(dev_bf16(Xc), cd, W13d, 128, L)
    Ac = gpu_lib.silu_mul(Gc)
    Yc = gpu_lib.expert_gemm_contiguous(Ac, cd, W2d, 128, L).cpu().numpy()
    for e, c in enumerate(counts_l):
        if c == 0:
            continue
        ym, yc = Ym[e, :c], Yc[starts[e]:starts[e] + c]
        assert np.array_equal(ym.view(np.uint32), yc.view(np.uint32)), f"expert {e}"
        g1 = oracle.contraction_ref(rows_e[e], W13[e])
        act = oracle.silu_mul_ref(g1[:, :I], g1[:, I:])
        assert_gemm_close(ym, oracle.contraction_ref(act, W2[e]), what=f"ffn expert {e}")


@pytest.mark.slow
def test_expert_gemm_moe_config(gpu_lib):
    """The MoE config's routed rows (4096 tokens, top-8, 64 experts, 2048 -> 1408)
    in both layouts: every row the same bits; sampled rows against the oracle."""
    cfg = wl.CONFIGS["moe"]
    s = wl.streams(cfg.seed)
    H = wl.normal_bf16(s["H"], (cfg.tokens, cfg.K), 1.0)
    We = wl.normal_bf16(s["W"], (cfg.experts, cfg.N, cfg.K), 0.02)
    ids, _ = wl.routing_input(s["route"], cfg.tokens, cfg.experts, cfg.topk)
    rows_e = [H[np.nonzero((ids == e).any(axis=1))[0]] for e in range(cfg.experts)]
    cap = int(-(-max(r.shape[0] for r in rows_e) // 64) * 64)
    counts, Xm, Xc, starts = _layouts(s["extra"], rows_e, cfg.K, cap, 128)
    say(f"expert gemm moe config: rows {int(counts.sum())} cap {cap}")
    Ym = _masked(gpu_lib, Xm, counts, We, cfg.leaves).cpu().numpy()
    Yc = _contig(gpu_lib, Xc, counts, We, 128, cfg.leaves).cpu().numpy()
    pick = s["perm"]
    for e, c in enumerate(counts.tolist()):
        ym, yc = Ym[e, :c], Yc[starts[e]:starts[e] + c]
        assert np.array_equal(ym.view(np.uint32), yc.view(np.uint32)), f"expert {e}"
        i = pick.choice(c, size=min(c, 8), replace=False)
        assert_gemm_close(ym[i], oracle.contraction_ref(rows_e[e][i], We[e]), what=f"expert {e}")
