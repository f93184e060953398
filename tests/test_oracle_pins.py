"""Pins for the CPU oracle: brute force, closed forms, invariants (no GPU).

Each test ties the oracle to something other than itself: exact rational
arithmetic on tiny inputs, integer arithmetic, hand-derived float32 closed
forms (tests/golden), and properties the mathematics fixes.  They are chosen so
that a dropped term, a wrong sign or index, a transposed operand, a wrong leaf
boundary or a wrong tree shape fails at least one of them.
"""

import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# helpers (independent of the oracle's own arithmetic)
# ---------------------------------------------------------------------------

def parse_dyadic(s: str) -> Fraction:
    """Parse '1+3*2^-23', '-2^24', '2^-3' into an exact Fraction."""
    s = s.replace(" ", "")
    total = Fraction(0)
    for sign, term in re.findall(r"([+-]?)([^+-]+(?:\^-?\d+)?)", s.replace("^-", "^~")):
        term = term.replace("^~", "^-")
        f = Fraction(1)
        for factor in term.split("*"):
            if "^" in factor:
                b, e = factor.split("^")
                f *= Fraction(int(b)) ** int(e)
            else:
                f *= Fraction(int(factor))
        total += -f if sign == "-" else f
    return total


def load_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([c.strip() for c in line.split("|")])
    return rows


def bf16_value_independent(bits: int) -> Fraction:
    """bf16 bit pattern -> exact value from sign / exponent / mantissa fields."""
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    assert e not in (0, 0xFF), "normal values only"
    v = Fraction(128 + m, 128) * Fraction(2) ** (e - 127)
    return -v if s else v


def f32_exact(f: Fraction) -> np.float32:
    x = np.float32(float(f))
    assert Fraction(float(x)) == f, "closed form is not a float32 value"
    return x


# ---------------------------------------------------------------------------
# bf16 storage
# ---------------------------------------------------------------------------

def test_bf16_decode_matches_field_formula():
    rng = np.random.default_rng(7)
    bits = wl.normal_bf16(rng, (4000,), std=3.0)
    got = oracle.bf16_bits_to_f64(bits)
    for b, g in zip(bits[:500], got[:500]):
        if b & 0x7FFF == 0:
            assert g == 0.0
            continue
        assert Fraction(float(g)) == bf16_value_independent(int(b))


def test_bf16_rounding_of_generator_is_nearest_even():
    # 1 + 2^-8 is halfway between bf16 1 and 1+2^-7: ties to the even (1).
    # 1 + 3*2^-8 is halfway between 1+2^-7 and 1+2^-6: ties to 1+2^-6.
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -2.5, 2**-24],
                 dtype=np.float32)
    got = wl.f32_to_bf16_bits(x)
    exp = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x3380]
    assert [int(v) for v in got] == exp


def test_sign_generator_gives_signed_powers_of_two():
    rng = np.random.default_rng(8)
    for e in (0, -12, 5):
        v = oracle.bf16_bits_to_f64(wl.sign_bf16(rng, (3, 700), e, chunk=257))
        assert np.all(np.abs(v) == 2.0 ** e)
        frac = np.mean(v > 0)
        assert 0.4 < frac < 0.6
    # the stream does not depend on the chunk size
    a = wl.sign_bf16(np.random.default_rng(9), (1000,), 0, chunk=1 << 24)
    b = wl.sign_bf16(np.random.default_rng(9), (1000,), 0, chunk=130)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# P1: brute force on tiny inputs with exact rational arithmetic
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_contraction_and_logprob_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    M, K, V = 3, 16, 8
    H = wl.normal_bf16(rng, (M, K), 1.0)
    W = wl.normal_bf16(rng, (V, K), 0.5)
    ids = rng.integers(0, V, size=M)
    Hq = [[bf16_value_independent(int(b)) if b & 0x7FFF else Fraction(0) for b in r] for r in H]
    Wq = [[bf16_value_independent(int(b)) if b & 0x7FFF else Fraction(0) for b in r] for r in W]
    X_exact = [[sum(h * w for h, w in zip(hr, wr)) for wr in Wq] for hr in Hq]

    X = oracle.contraction_ref(H, W)
    assert X.shape == (M, V)
    for m in range(M):
        for v in range(V):
            assert abs(X[m, v] - float(X_exact[m][v])) <= 1e-12 * (1 + abs(float(X_exact[m][v])))

    lp, lse = oracle.logprob_ref(H, W, ids)
    for m in range(M):
        xs = [float(x) for x in X_exact[m]]
        g = max(xs)
        lse_bf = g + math.log(math.fsum(math.exp(x - g) for x in xs))
        assert abs(lse[m] - lse_bf) <= 1e-12 * (1 + abs(lse_bf))
        assert abs(lp[m] - (xs[ids[m]] - lse_bf)) <= 1e-12 * (1 + abs(lse_bf))


def test_contraction_exact_integers_not_transposed():
    # Small integers: every partial sum is an integer, so float64 is exact and
    # must equal int64 arithmetic; M != N != K catches a transposed operand.
    rng = np.random.default_rng(3)
    A = wl.integer_bf16(rng, (5, 24), -3, 3)
    W = wl.integer_bf16(rng, (7, 24), -3, 3)
    Ai = oracle.bf16_bits_to_f64(A).astype(np.int64)
    Wi = oracle.bf16_bits_to_f64(W).astype(np.int64)
    expect = np.einsum("mk,nk->mn", Ai, Wi)
    got = oracle.contraction_ref(A, W)
    assert np.array_equal(got, expect.astype(np.float64))


def test_contraction_row_chunking_changes_nothing():
    rng = np.random.default_rng(4)
    A = wl.normal_bf16(rng, (37, 64))
    W = wl.normal_bf16(rng, (11, 64), 0.02)
    assert np.array_equal(oracle.contraction_ref(A, W, row_chunk=5),
                          oracle.contraction_ref(A, W, row_chunk=1000))


# ---------------------------------------------------------------------------
# P2: invariants of the log-softmax and the logprob
# ---------------------------------------------------------------------------

def test_log_softmax_invariants():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((6, 50)) * 4
    L = oracle.log_softmax_ref(X)
    assert np.allclose(oracle.lse_ref(L), 0.0, atol=1e-12)          # logsumexp of log-softmax
    assert np.allclose(np.exp(L).sum(axis=1), 1.0, atol=1e-12)       # softmax sums to one
    assert np.allclose(oracle.log_softmax_ref(X + 123.25), L, atol=1e-12)  # shift invariance
    assert np.all(L <= 0)
    # overflow-safe: equal huge logits give exactly log(V) above the logit
    big = np.full((1, 4), 1000.0)
    assert abs(oracle.lse_ref(big)[0] - (1000.0 + math.log(4))) < 1e-12


def test_logprob_row_and_vocab_permutation():
    rng = np.random.default_rng(6)
    M, K, V = 9, 32, 40
    H = wl.normal_bf16(rng, (M, K))
    W = wl.normal_bf16(rng, (V, K), 0.1)
    ids = rng.integers(0, V, size=M)
    lp, _ = oracle.logprob_ref(H, W, ids)
    # rows: permuting the batch permutes the outputs (each row stands alone)
    p = rng.permutation(M)
    lp_p, _ = oracle.logprob_ref(H[p], W, ids[p])
    assert np.array_equal(lp_p, lp[p])
    # vocabulary: permute W's rows and remap ids; logprobs are unchanged
    q = rng.permutation(V)
    inv = np.empty(V, dtype=np.int64)
    inv[q] = np.arange(V)
    lp_q, _ = oracle.logprob_ref(H, W[q], inv[ids])
    assert np.allclose(lp_q, lp, atol=1e-12)
    # one row alone equals the same row inside the batch
    for r in (0, 4, 8):
        one, _ = oracle.logprob_ref(H[r:r + 1], W, ids[r:r + 1])
        assert abs(one[0] - lp[r]) <= 1e-12


# ---------------------------------------------------------------------------
# P5 / P6: closed forms and special cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("V", [1, 7, 4096, 151936])
def test_equal_logits_give_minus_log_V(V):
    K = 8
    rng = np.random.default_rng(V)
    H = wl.normal_bf16(rng, (2, K))
    row = wl.normal_bf16(rng, (1, K), 0.5)
    W = np.repeat(row, V, axis=0)
    ids = np.array([0, V - 1])
    lp, _ = oracle.logprob_ref(H, W, ids)
    assert np.allclose(lp, -math.log(V), atol=1e-12)
    Wz = np.zeros((V, K), dtype=np.uint16)   # W = 0: all logits 0
    lpz, lsez = oracle.logprob_ref(H, Wz, ids)
    assert np.allclose(lpz, -math.log(V), atol=1e-12)
    assert np.allclose(lsez, math.log(V), atol=1e-12)


def test_one_distinct_logit_closed_form():
    V, K, a = 1000, 4, 2.5
    H = wl.f32_to_bf16_bits(np.array([[1.0, 0, 0, 0]], dtype=np.float32))
    Wf = np.zeros((V, K), dtype=np.float32)
    Wf[17, 0] = a
    W = wl.f32_to_bf16_bits(Wf)
    lp, _ = oracle.logprob_ref(H, W, np.array([17]))
    assert abs(lp[0] - (a - math.log(math.exp(a) + V - 1))) < 1e-12
    lp0, _ = oracle.logprob_ref(H, W, np.array([3]))
    assert abs(lp0[0] - (0 - math.log(math.exp(a) + V - 1))) < 1e-12


def test_one_hot_row_reads_a_column_of_W():
    rng = np.random.default_rng(8)
    K, V = 16, 30
    W = wl.normal_bf16(rng, (V, K), 0.3)
    Hf = np.zeros((1, K), dtype=np.float32)
    Hf[0, 11] = 1.0
    X = oracle.contraction_ref(wl.f32_to_bf16_bits(Hf), W)
    assert np.array_equal(X[0], oracle.bf16_bits_to_f64(W[:, 11]))


def test_invalid_id_is_nan_for_that_row_only():
    rng = np.random.default_rng(9)
    H = wl.normal_bf16(rng, (4, 8))
    W = wl.normal_bf16(rng, (5, 8))
    lp, lse = oracle.logprob_ref(H, W, np.array([0, -1, 5, 4]))
    assert np.isfinite(lp[0]) and np.isfinite(lp[3])
    assert np.isnan(lp[1]) and np.isnan(lp[2])
    assert np.all(np.isfinite(lse))


# ---------------------------------------------------------------------------
# Fixed binary tree in float32 (closed forms in tests/golden)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("row", load_golden("tree_f32_closed_forms.txt"), ids=lambda r: r[0])
def test_leaf_tree_closed_forms(row):
    name, leaves, expected, _why = row
    P = np.array([f32_exact(parse_dyadic(v)) for v in leaves.split(",")], dtype=np.float32)
    got = oracle.leaf_tree_f32(P)
    assert got.dtype == np.float32
    assert Fraction(float(got)) == parse_dyadic(expected)


def test_leaf_tree_closed_forms_have_power():
    """The golden leaves separate the tree from plausible wrong schedules."""
    rows = {r[0]: r for r in load_golden("tree_f32_closed_forms.txt")}
    P = [f32_exact(parse_dyadic(v)) for v in rows["L8_adjacent"][1].split(",")]
    seq = np.float32(0)
    for p in P:
        seq = np.float32(seq + p)
    assert seq != oracle.leaf_tree_f32(np.array(P))
    Q = [f32_exact(parse_dyadic(v)) for v in rows["L8_not_strided"][1].split(",")]
    strided = [np.float32(Q[i] + Q[i + 4]) for i in range(4)]
    strided = np.float32(np.float32(strided[0] + strided[2]) + np.float32(strided[1] + strided[3]))
    assert strided != oracle.leaf_tree_f32(np.array(Q))


@pytest.mark.parametrize("where", ["start", "end"])
@pytest.mark.parametrize("leaves,K", [(8, 512), (16, 7168), (8, 64)])
def test_leaf_tree_gemm_leaf_boundaries(where, leaves, K):
    """One nonzero product per leaf: the leaf sums are exact, only the tree rounds."""
    golden = {r[0]: r for r in load_golden("tree_f32_closed_forms.txt")}
    key = "L8_adjacent" if leaves == 8 else "L16_adjacent"
    vals = [f32_exact(parse_dyadic(v)) for v in golden[key][1].split(",")]
    ell = K // leaves
    A = np.zeros((2, K), dtype=np.float32)
    W = np.zeros((3, K), dtype=np.float32)
    for l in range(leaves):
        k = l * ell if where == "start" else (l + 1) * ell - 1
        A[:, k] = 1.0
        W[1, k] = vals[l]
    got = oracle.leaf_tree_gemm_f32(wl.f32_to_bf16_bits(A), wl.f32_to_bf16_bits(W), leaves)
    assert got.dtype == np.float32 and got.shape == (2, 3)
    assert np.all(got[:, [0, 2]] == 0)
    assert np.all(np.array([Fraction(float(x)) for x in got[:, 1]]) == parse_dyadic(golden[key][2]))


def test_leaf_tree_gemm_integers_equal_exact():
    rng = np.random.default_rng(10)
    A = wl.integer_bf16(rng, (6, 128), -4, 4)
    W = wl.integer_bf16(rng, (5, 128), -4, 4)
    got = oracle.leaf_tree_gemm_f32(A, W, 8)
    assert np.array_equal(got.astype(np.float64), oracle.contraction_ref(A, W))


def test_leaf_bounds_rejects_bad_counts():
    with pytest.raises(ValueError):
        oracle.leaf_bounds(96, 3)
    with pytest.raises(ValueError):
        oracle.leaf_bounds(100, 8)
    assert oracle.leaf_bounds(64, 4) == [(0, 16), (16, 32), (32, 48), (48, 64)]


# ---------------------------------------------------------------------------
# MoE: fp64 definition and the float32 fixed-order combine
# ---------------------------------------------------------------------------

def test_moe_ref_brute_force():
    rng = np.random.default_rng(11)
    T, E, N, K, topk = 4, 5, 3, 8, 2
    H = wl.normal_bf16(rng, (T, K))
    We = wl.normal_bf16(rng, (E, N, K), 0.5)
    ids, w = wl.routing_input(rng, T, E, topk)
    got = oracle.moe_ref(H, We, ids, w)
    for t in range(T):
        for n in range(N):
            acc = Fraction(0)
            for s in range(topk):
                e = ids[t, s]
                y = sum(bf16_value_independent(int(h)) * bf16_value_independent(int(x))
                        for h, x in zip(H[t], We[e, n]) if h & 0x7FFF and x & 0x7FFF)
                acc += Fraction(float(w[t, s])) * y
            assert abs(got[t, n] - float(acc)) <= 1e-12 * (1 + abs(float(acc)))


def test_moe_top1_unit_gate_is_the_contraction():
    rng = np.random.default_rng(12)
    T, E, N, K = 6, 3, 4, 16
    H = wl.normal_bf16(rng, (T, K))
    We = wl.normal_bf16(rng, (E, N, K), 0.1)
    ids = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    w = np.ones((T, 1), dtype=np.float32)
    got = oracle.moe_ref(H, We, ids, w)
    for t in range(T):
        assert np.array_equal(got[t], oracle.contraction_ref(H[t:t + 1], We[ids[t, 0]])[0])


@pytest.mark.parametrize("row", load_golden("moe_combine_closed_forms.txt"), ids=lambda r: r[0])
def test_moe_combine_closed_forms(row):
    name, ids, gates, ys, expected, _why = row
    ids = np.array([[int(v) for v in ids.split(",")]])
    w = np.array([[f32_exact(parse_dyadic(v)) for v in gates.split(",")]], dtype=np.float32)
    Y = np.array([[[f32_exact(parse_dyadic(v))] for v in ys.split(",")]], dtype=np.float32)
    got = oracle.moe_combine_f32(Y, ids, w)
    assert got.shape == (1, 1) and got.dtype == np.float32
    assert Fraction(float(got[0, 0])) == parse_dyadic(expected)


def test_routing_input_is_valid():
    rng = np.random.default_rng(13)
    ids, w = wl.routing_input(rng, 2000, 64, 8)
    assert ids.shape == (2000, 8) and ids.dtype == np.int32 and w.dtype == np.float32
    for r in ids:
        assert len(set(r.tolist())) == 8 and r.min() >= 0 and r.max() < 64
    assert np.all(w > 0) and np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    # every expert is used about equally (16000 pairs over 64 experts: 250 each)
    cnt = np.bincount(ids.reshape(-1), minlength=64)
    assert cnt.min() > 150 and cnt.max() < 350


# ---------------------------------------------------------------------------
# The router   [Bit-consistent RL, sections 1 and 4.1; reading R13]
# ---------------------------------------------------------------------------

def _rank_select(row, k):
    """Brute force: rank(e) = #{better e'}, better = larger value, or equal value
    and lower id; NaN after every number, NaNs by id.  Slot r holds rank r."""
    def better(a, b):   # is expert a ahead of expert b?
        va, vb = row[a], row[b]
        na, nb = math.isnan(va), math.isnan(vb)
        if na or nb:
            return (not na and nb) or (na and nb and a < b)
        return va > vb or (va == vb and a < b)
    E = len(row)
    rank = [sum(better(o, e) for o in range(E) if o != e) for e in range(E)]
    assert sorted(rank) == list(range(E))
    return [rank.index(r) for r in range(k)]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_route_select_brute_force_ranks(seed):
    rng = np.random.default_rng(700 + seed)
    E, k = 12, 5
    X = rng.integers(-2, 3, size=(40, E)).astype(np.float64)   # many ties
    X[0, [1, 4, 7]] = [0.0, -0.0, 0.0]                            # signed zeros tie
    X[1] = -0.0
    X[2, 3] = np.nan
    X[3, :] = np.nan
    X[3, 9] = -5.0
    got = oracle.route_select(X, k)
    for t in range(X.shape[0]):
        assert got[t].tolist() == _rank_select(X[t].tolist(), k), t


def test_route_equal_logits_take_lowest_ids_with_equal_gates():
    X = np.full((3, 64), 0.75)
    ids = oracle.route_select(X, 8)
    assert np.all(ids == np.arange(8))
    assert np.all(oracle.route_gates_ref(X, ids) == 1.0 / 8)


def test_route_gates_closed_form():
    # logits 0, -ln 2, -2 ln 2, -3 ln 2 and far smaller ones: exp terms 1, 1/2,
    # 1/4, 1/8 of sum 15/8, so the gates are 8/15, 4/15, 2/15, 1/15
    ln2 = math.log(2.0)
    row = np.array([-9.0, -ln2, -20.0, 0.0, -3 * ln2, -2 * ln2, -30.0, -11.0])
    ids = oracle.route_select(row[None], 4)
    assert ids[0].tolist() == [3, 1, 5, 4]
    g = oracle.route_gates_ref(row[None], ids)[0]
    assert np.allclose(g, [8 / 15, 4 / 15, 2 / 15, 1 / 15], rtol=0, atol=1e-15)


def test_route_gates_invariants():
    rng = np.random.default_rng(711)
    X = rng.standard_normal((50, 64))
    ids = oracle.route_select(X, 8)
    g = oracle.route_gates_ref(X, ids)
    assert np.allclose(g.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(np.diff(g, axis=1) <= 0)                      # largest logit first
    assert np.allclose(oracle.route_gates_ref(X + 3.5, ids), g, atol=1e-14)
    top1 = oracle.route_select(X, 1)[:, 0]
    assert np.all(top1 == np.argmax(X, axis=1))                 # argmax takes the first maximum
    assert np.all(oracle.route_gates_ref(X, top1[:, None]) == 1.0)


def test_route_ref_is_the_contraction_then_the_rule():
    rng = np.random.default_rng(712)
    H = wl.integer_bf16(rng, (9, 64), -2, 2)
    Wr = wl.integer_bf16(rng, (16, 64), -2, 2)
    logits, ids, g = oracle.route_ref(H, Wr, 4)
    exact = oracle.as_f64(H) @ oracle.as_f64(Wr).T                # small integers: exact
    assert np.array_equal(logits, exact)
    for t in range(9):
        assert ids[t].tolist() == _rank_select(exact[t].tolist(), 4)


# ---------------------------------------------------------------------------
# Deterministic Top-K of positions   [Bit-consistent RL, section 4.3]
# ---------------------------------------------------------------------------

def _topk_brute(row, n, k):
    """Rank counting: p is ahead of q when score(p) > score(q), or equal scores
    and p > q; NaN after every number (NaNs: larger position first)."""
    def ahead(p, q):
        a, b = row[p], row[q]
        na, nb = math.isnan(a), math.isnan(b)
        if na or nb:
            return (not na and nb) or (na and nb and p > q)
        return a > b or (a == b and p > q)
    sel = [p for p in range(n) if sum(ahead(q, p) for q in range(n) if q != p) < k]
    sel = sorted(sel, reverse=True)
    return sel + [-1] * (k - len(sel))


def test_topk_golden_examples():
    for name, k, n, pairs, expect in load_golden("topk_figure_example.txt"):
        k, n = int(k), int(n)
        row = np.full((1, max(n, 64)), -1.0)
        for item in [x for x in pairs.split(",") if x.strip()]:
            p, v = item.split("=")
            row[0, int(p)] = float(Fraction(v.strip()))
        if not pairs.strip():
            row[0, :] = 0.5
        got = oracle.topk_positions(row, [n], k)[0].tolist()
        assert got == [int(x) for x in expect.split(",")], name
        assert got == _topk_brute(row[0].tolist(), n, k), name


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_topk_positions_brute_force(seed):
    rng = np.random.default_rng(800 + seed)
    R, N, k = 12, 40, 7
    S = rng.integers(-3, 4, size=(R, N)).astype(np.float64)        # many ties
    S[0, 5:9] = [0.0, -0.0, 0.0, -0.0]
    S[1, :] = np.nan
    S[1, [3, 30]] = [-7.0, 2.0]
    S[2, ::3] = np.nan
    lengths = rng.integers(0, N + 1, size=R)
    lengths[:3] = N
    lengths[3] = 0
    lengths[4] = 5                                                   # fewer than k
    got = oracle.topk_positions(S, lengths, k)
    for r in range(R):
        assert got[r].tolist() == _topk_brute(S[r].tolist(), int(lengths[r]), k), r


def test_topk_positions_properties():
    rng = np.random.default_rng(810)
    S = rng.standard_normal((5, 3000))
    lengths = np.array([3000, 2999, 2048, 100, 1])
    out = oracle.topk_positions(S, lengths, 2048)
    for r in range(5):
        n = int(lengths[r])
        sel = out[r][out[r] >= 0]
        assert sel.size == min(2048, n) and np.all(out[r][sel.size:] == -1)
        assert np.all(np.diff(sel) < 0)                                   # descending positions
        if sel.size < n:
            rest = np.setdiff1d(np.arange(n), sel)
            assert S[r, sel].min() >= S[r, rest].max()                    # the largest scores


# ---------------------------------------------------------------------------
# Gumbel-max sampling and the k3 metric
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# Expert layouts and the activation between the expert GEMMs
#   [Bit-consistent RL, section 4.4]
# ---------------------------------------------------------------------------

def _bf16_value(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern from its fields."""
    sign = -1 if bits & 0x8000 else 1
    ex, man = (bits >> 7) & 0xFF, bits & 0x7F
    if ex == 0:
        return sign * Fraction(man, 1 << 7) * Fraction(1, 1 << 126)
    return sign * (1 + Fraction(man, 1 << 7)) * (Fraction(2) ** (ex - 127))


def _bf16_round_exact(x: Fraction) -> int:
    """Nearest bf16 to the rational x (halves to the even pattern), by looking
    at the patterns around it: independent of any floating-point rounding."""
    if x == 0:
        return 0
    neg = x < 0
    a = -x if neg else x
    # the largest non-negative pattern not above a (patterns of one sign are ordered)
    lo, hi = 0, 0x7F7F
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if _bf16_value(mid) <= a:
            lo = mid
        else:
            hi = mid - 1
    if lo == 0x7F7F:
        half = (_bf16_value(0x7F7F) - _bf16_value(0x7F7E)) / 2
        b = 0x7F80 if a >= _bf16_value(0x7F7F) + half else 0x7F7F
    else:
        d0, d1 = a - _bf16_value(lo), _bf16_value(lo + 1) - a
        b = lo if d0 < d1 else (lo + 1 if d1 < d0 else (lo if lo % 2 == 0 else lo + 1))
    return b | (0x8000 if neg else 0)


def test_f64_to_bf16_fixed_points():
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -30, -2.5, 0.0, -0.0,
                  1e-40, np.inf, -np.inf, 3.39e38, 3.4e38])
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000, 0x8000, 0x0001, 0x7F80, 0xFF80, 0x7F7F, 0x7F80]
    assert oracle.f64_to_bf16_rne(x).tolist() == want
    # one rounding: through float32 first, 1 + 2^-8 + 2^-30 would become the tie 1 + 2^-8 and then 1.0
    assert np.float32(1 + 2.0 ** -8 + 2.0 ** -30) == np.float32(1 + 2.0 ** -8)
    assert oracle.f64_to_bf16_rne(np.array([np.nan]))[0] & 0x7FFF > 0x7F80


def test_f64_to_bf16_matches_exact_rounding():
    rng = np.random.default_rng(1900)
    x = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-40, 38, 300),
                        rng.standard_normal(50) * 1e-39])
    got = oracle.f64_to_bf16_rne(x)
    for v, b in zip(x.tolist(), got.tolist()):
        assert b == _bf16_round_exact(Fraction(v)), v


def _silu_mul_decimal(g: float, u: float) -> Fraction:
    import decimal
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        dg = decimal.Decimal(g)
        val = dg / (1 + (-dg).exp()) * decimal.Decimal(u)
    return Fraction(val)


def test_silu_mul_against_high_precision():
    """SiLU(g)*u from 60-digit decimal arithmetic, rounded exactly: the oracle
    agrees except where the value lies within 1e-12 (relative) of a rounding
    midpoint, which no case here does."""
    rng = np.random.default_rng(1901)
    g = np.concatenate([rng.standard_normal(400) * 3, [0.0, 30.0, -30.0, 80.0, -80.0, 1e-3]])
    u = np.concatenate([rng.standard_normal(400) * 2, [1.5, -1.0, 1.0, 0.5, 2.0, -7.0]])
    got = oracle.silu_mul_ref(g, u)
    checked = 0
    for gi, ui, b in zip(g.tolist(), u.tolist(), got.tolist()):
        exact = _silu_mul_decimal(gi, ui)
        r = _bf16_round_exact(exact)
        if r & 0x7FFF not in (0, 0x7F80):
            nb = r + 1 if (exact > 0) == (r < 0x8000) else r - 1
            mid = (_bf16_value(r) + _bf16_value(nb)) / 2
            if abs(exact - mid) <= abs(exact) * Fraction(1, 10 ** 12):
                continue
        assert b == r, (gi, ui, hex(b), hex(r))
        checked += 1
    assert checked >= 400


def test_silu_mul_closed_forms():
    ln3 = math.log(3.0)
    # sigma(ln 3) = 3/4: SiLU(ln 3) = 0.75 ln 3 = 0.82396...; bf16 step on [0.5, 1) is 2^-8: 211/256
    b = oracle.silu_mul_ref(np.array([ln3]), np.array([1.0]))[0]
    assert _bf16_value(int(b)) == Fraction(211, 256)
    z = oracle.silu_mul_ref(np.array([0.0, 0.0]), np.array([5.0, -5.0]))
    assert z.tolist() == [0x0000, 0x8000]                    # 0 * u keeps the sign of u
    big = oracle.silu_mul_ref(np.array([100.0, -100.0]), np.array([1.0, 1.0]))
    assert big[0] == 0x42C8                                  # SiLU(100) = 100 to far below a bf16 step
    # SiLU(-100) = -100 e^-100 = -3.7e-42, below half the smallest bf16 subnormal (2^-134): -0
    assert big[1] == 0x8000
    # SiLU(-95) = -95 e^-95 = -5.5e-40 = -6.0 steps of 2^-133: the subnormal pattern 6
    assert oracle.silu_mul_ref(np.array([-95.0]), np.array([1.0]))[0] == 0x8006


def test_silu_mul_rounds_once_not_twice():
    """Rounding SiLU to bf16 before the multiply changes some results by one
    step (the section's point); the oracle follows the one rounding."""
    rng = np.random.default_rng(1902)
    g = rng.standard_normal(2000) * 2
    u = np.full(2000, 3.0)
    once = oracle.silu_mul_ref(g, u)
    silu = g / (1.0 + np.exp(-g))
    twice = oracle.f64_to_bf16_rne(oracle.bf16_bits_to_f64(oracle.f64_to_bf16_rne(silu)) * 3.0)
    diff = np.flatnonzero(once != twice)
    assert diff.size > 20
    for i in diff[:20]:
        assert once[i] == _bf16_round_exact(_silu_mul_decimal(float(g[i]), 3.0))


def test_expert_row_starts_closed_forms():
    s, r = oracle.expert_row_starts([3, 0, 130, 1], "contiguous", align=128)
    assert s.tolist() == [0, 128, 128, 384] and r.tolist() == [3, 0, 130, 1]
    s, r = oracle.expert_row_starts([3, 0, 130, 1], "contiguous", align=1)
    assert s.tolist() == [0, 3, 3, 133]
    s, r = oracle.expert_row_starts([3, 0, 130, 1, -2], "masked", cap=100)
    assert s.tolist() == [0, 100, 200, 300, 400] and r.tolist() == [3, 0, 100, 1, 0]


def test_expert_gemm_ref_brute_force():
    rng = np.random.default_rng(1903)
    E, N, K = 3, 5, 6
    W = wl.integer_bf16(rng, (E, N, K), -3, 3)
    for layout, cap, align in (("masked", 4, 1), ("contiguous", 0, 4), ("contiguous", 0, 1)):
        counts = [2, 0, 4]
        starts, rows = oracle.expert_row_starts(counts, layout, cap, align)
        M = int(max(starts + np.maximum(rows, 1)))
        X = wl.integer_bf16(rng, (M, K), -4, 4)
        Y = oracle.expert_gemm_ref(X, counts, W, layout, cap, align)
        owner = {}
        for e in range(E):
            for i in range(int(rows[e])):
                owner[int(starts[e]) + i] = e
        Xv = oracle.bf16_bits_to_f64(X)
        Wv = oracle.bf16_bits_to_f64(W)
        for m in range(M):
            if m not in owner:
                assert np.all(np.isnan(Y[m]))
                continue
            for n in range(N):
                exact = sum(Fraction(Xv[m, k]) * Fraction(Wv[owner[m], n, k]) for k in range(K))
                assert Y[m, n] == exact


# ---------------------------------------------------------------------------
# Block FP8 (W8A8)   [Bit-consistent RL, sections 4.1 and 4.4]
# ---------------------------------------------------------------------------

def _e4m3_exact(code: int) -> Fraction:
    """Value of an E4M3 byte from its fields, as a rational."""
    sign = -1 if code & 0x80 else 1
    ex, man = (code >> 3) & 0xF, code & 0x7
    if ex == 0:
        return sign * Fraction(man, 8) * Fraction(1, 64)
    return sign * (1 + Fraction(man, 8)) * Fraction(2) ** (ex - 7)


def test_e4m3_codes_round_trip():
    codes = [c for c in range(256) if c & 0x7F != 0x7F]          # every code but NaN
    vals = oracle.e4m3_value(np.array(codes, dtype=np.uint8))
    for c, v in zip(codes, vals.tolist()):
        assert Fraction(v) == _e4m3_exact(c), c
    back = oracle.f64_to_e4m3_rne(vals)
    assert back.tolist() == codes                                  # -0 keeps its sign bit
    assert oracle.e4m3_value(np.array([0x7E]))[0] == 448.0 and np.isnan(oracle.e4m3_value(np.array([0xFF]))[0])


def test_e4m3_rounding_is_nearest_even():
    """Against the exact nearest of all finite codes, halves to the even mantissa."""
    rng = np.random.default_rng(2000)
    x = np.concatenate([rng.uniform(-448, 448, 300), rng.uniform(-2.0 ** -5, 2.0 ** -5, 200),
                        [232.0, 1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11, 447.9, -0.0]])
    finite = [c for c in range(128) if c != 0x7F]
    got = oracle.f64_to_e4m3_rne(x)
    for v, b in zip(x.tolist(), got.tolist()):
        a = abs(Fraction(v))
        best = min(finite, key=lambda c: (abs(_e4m3_exact(c) - a), c & 1))
        assert b & 0x7F == best, (v, b, best)
        assert (b >> 7) == (1 if math.copysign(1.0, v) < 0 else 0)
    with pytest.raises(ValueError):
        oracle.f64_to_e4m3_rne(np.array([449.0]))


def test_fp8_block_exponent_closed_forms():
    from oracle.reference import _block_exponent
    amax = np.array([448.0, 449.0, 1.0, 0.0, 0.875, 896.0, 1.75, 1.7501, 3e-5, 2.0 ** -126, 3.3895e38])
    # 448 2^e >= amax > 448 2^(e-1): hand-derived (448 = 1.75 * 2^8); 2^-126 would need e = -134,
    # below the E8M0 floor of -127; the largest bf16, (2 - 2^-7) 2^127, needs 120
    assert _block_exponent(amax).tolist() == [0, 1, -8, 0, -9, 1, -8, -7, -23, -127, 120]


def test_fp8_block_quant_hand_example():
    """Blocks of 1 x 2: [1, -3] has amax 3, e = -7 (448/128 = 3.5 >= 3 > 1.75): 128 and -384
    = codes 0x70 and 0xFC; [500, 0] has e = 1: 250 rounds to 256 (6 away, not 10) = 0x78."""
    q, e = oracle.fp8_block_quant(np.array([[1.0, -3.0, 500.0, 0.0]]), 1, 2)
    assert q.tolist() == [[0x70, 0xFC, 0x78, 0x00]] and e.tolist() == [[-7, 1]]
    assert oracle.fp8_dequant(q, e, 1, 2).tolist() == [[1.0, -3.0, 512.0, 0.0]]


def test_fp8_blocks_are_independent_and_bounded():
    rng = np.random.default_rng(2001)
    W = wl.normal_bf16(rng, (300, 260), 0.02)                      # cut blocks at both edges
    q, e = oracle.fp8_block_quant(W, 128, 128)
    assert q.shape == (300, 260) and e.shape == (3, 3)
    W2 = W.copy()
    W2[130:140, 5:9] = wl.normal_bf16(rng, (10, 4), 3.0)           # only block (1, 0) changes
    q2, e2 = oracle.fp8_block_quant(W2, 128, 128)
    same = np.ones((300, 260), bool)
    same[128:256, 0:128] = False
    assert np.array_equal(q[same], q2[same]) and e2[1, 0] != e[1, 0]
    assert np.array_equal(np.delete(e.ravel(), 3), np.delete(e2.ravel(), 3))
    # each element within half an E4M3 step of x * 2^-e (relative 2^-4 above 2^-6)
    x = oracle.bf16_bits_to_f64(W)
    ee = np.repeat(np.repeat(e, 128, 0), 128, 1)[:300, :260]
    t = np.ldexp(x, -ee)
    err = np.abs(oracle.e4m3_value(q) - t)
    assert np.all((err <= np.abs(t) * 2.0 ** -4) | (err <= 2.0 ** -10))
    assert np.all(np.abs(t) <= 448.0)


def test_fp8_gemm_ref_brute_force():
    rng = np.random.default_rng(2002)
    A = wl.normal_bf16(rng, (3, 256), 1.0)
    W = wl.normal_bf16(rng, (5, 256), 0.02)
    qa, ea = oracle.fp8_block_quant(A, 1)
    qw, ew = oracle.fp8_block_quant(W, 128)
    C = oracle.fp8_gemm_ref(qa, ea, qw, ew)
    for m in range(3):
        for n in range(5):
            exact = sum(_e4m3_exact(int(qa[m, k])) * Fraction(2) ** int(ea[m, k // 128]) *
                        _e4m3_exact(int(qw[n, k])) * Fraction(2) ** int(ew[0, k // 128]) for k in range(256))
            assert abs(Fraction(C[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


def test_gumbel_max_samples_the_softmax():
    rng = np.random.default_rng(14)
    n = 200_000
    X = np.tile(np.log(np.array([1.0, 2.0, 3.0, 4.0])), (n, 1))
    ids = oracle.gumbel_max_ids(X, wl.gumbel(rng, X.shape))
    freq = np.bincount(ids, minlength=4) / n
    assert np.allclose(freq, [0.1, 0.2, 0.3, 0.4], atol=0.005)
    Y = np.zeros((3, 5))
    Y[:, 2] = 60.0
    assert np.all(oracle.gumbel_max_ids(Y, wl.gumbel(rng, Y.shape)) == 2)


def test_k3_kl():
    a = np.array([-1.0, -2.0, -0.5])
    assert oracle.k3_kl(a, a) == 0.0
    d = 1e-3
    assert abs(oracle.k3_kl(a, a + d) - d * d / 2) < 1e-9
    assert oracle.k3_kl(a, a - 0.3) > 0
