"""fp64 / float32-emulating CPU oracle for the batch-invariant token-logprob path.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
``cpu_baseline`` leg of ``bench.py``; never by the product path.  It shares no
code with the HIP library or its Python binding.

Sources (the three web pages this method is described on):

* [IsoExec] "IsoExec: Unified Execution to Eliminate Trainer-Inference
  Mismatch in SkyRL", section "Parallelism-invariant kernels" and its figure of
  the fixed binary reduction tree: the contraction dimension K is cut into N
  contiguous leaves, each leaf is a deterministic matrix-core product with FP32
  accumulation, and the leaves are combined by a fixed binary schedule.  The
  contract example in "Unified execution contract" pins ``leaves = 8`` and an
  FP32 leaf dtype.
* [Bit-consistent RL] "Termina el entrenamiento RL más rápido: Consistente a
  nivel de bits, de alto rendimiento y dirigido por agentes", section 2 (diff is
  the per-sampled-token logprob difference and must be exactly zero; batch
  independence and phase consistency), section 4.4 (per-row expert GEMM result
  independent of layout) and section 4.5 (expert outputs summed in FP32 in a
  fixed order on the token's owner).

Readings where the pages leave a step open:

* R1 tree shape: a balanced tree of adjacent pairs, level by level, over a
  power-of-two leaf count: for 8 leaves ``((P0+P1)+(P2+P3))+((P4+P5)+(P6+P7))``.
* R5 the logits stay FP32 (the tree output) before the softmax.
* R6 the log-softmax is max-shifted: ``lse = g + log(sum(exp(x - g)))``.
* R8 a sampled id outside ``[0, V)`` yields NaN for that row only.
* R12 the MoE combine runs in ascending expert id, ``acc = acc + g*y`` with a
  float32 multiply then a float32 add, each rounded to nearest even.
* R19 the two expert layouts of section 4.4: masked = a block of ``cap`` rows
  per expert, expert e's rows at ``e*cap .. e*cap+count_e-1`` (counts above
  ``cap`` keep their first ``cap`` rows); contiguous = the experts' rows packed
  in expert order, each expert's segment starting at a multiple of ``align``
  (the alignment padding of the section's figure; ``align = 1`` packs them).
  The output of a row sits at the same row index as its input.
* R20 the activation between the two expert GEMMs (section 4.4, condition 3):
  ``SiLU(g) * u`` with ``SiLU(g) = g / (1 + exp(-g))``, computed exactly here
  and rounded to bf16 once, to nearest even; FP8 quantisation after it is not
  modelled (out of scope).
* R21 block FP8 (section 4.1: BF16 master weights quantised to block FP8 by
  the deployment rule, W8A8; section 4.4: per-element round to nearest): OCP
  E4M3 values (largest 448); a power-of-two scale 2^e per block, e the
  smallest integer >= -127 with amax <= 448 * 2^e (e = 0 for an all-zero
  block; -127 is the lowest exponent of the one-byte E8M0 scale encoding);
  each element is x * 2^-e rounded to E4M3 once, to nearest even.  Weight
  blocks are 128 x 128 (rows x columns of W), activation blocks 1 x 128 (a
  token's 128 consecutive columns); a block cut by the matrix edge takes the
  elements it has.  The product of two dequantised values is exact in FP32,
  so the W8A8 GEMM is the leaf-tree contraction of the dequantised values.
* R13 the router: logits are the FP32 leaf-tree contraction of the token with
  the router weight, the same at every batch size ([Bit-consistent RL],
  section 4.1: the router gate uses one FP32-output GEMM at every batch size);
  the top-k experts are taken largest logit first, equal logits in ascending
  expert id (the pages ask only that tie-breaking and output order be fixed,
  section 1); the gates are the softmax over the selected logits.

Parity status:

* ``contraction_ref``, ``lse_ref``, ``log_softmax_ref``, ``logprob_ref``,
  ``moe_ref``, ``route_select``, ``route_gates_ref``, ``route_ref``,
  ``topk_positions``, ``expert_row_starts``, ``expert_gemm_ref``,
  ``silu_mul_ref``, ``f64_to_bf16_rne``, ``e4m3_value``, ``f64_to_e4m3_rne``,
  ``fp8_block_quant``, ``fp8_dequant``, ``fp8_gemm_ref``: plain
  definitions in fp64; pinned by brute force (exact rational arithmetic, rank
  counting), closed forms and invariants in ``tests/test_oracle_pins.py``.
* ``leaf_tree_f32``, ``leaf_tree_gemm_f32``, ``moe_combine_f32``: float32
  emulators of the fixed orders; pinned by hand-derived closed forms.  They are
  exact models of the GPU only where every leaf sum (or every expert output) is
  itself exact in float32; elsewhere the rounding inside one leaf, which the
  matrix-core instruction performs, is not modelled ("parity unpinned" beyond
  the tolerance).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "as_f64",
    "leaf_bounds",
    "contraction_ref",
    "leaf_tree_f32",
    "leaf_tree_gemm_f32",
    "lse_ref",
    "log_softmax_ref",
    "logprob_ref",
    "gumbel_max_ids",
    "moe_ref",
    "moe_combine_f32",
    "route_select",
    "route_gates_ref",
    "route_ref",
    "topk_positions",
    "f64_to_bf16_rne",
    "expert_row_starts",
    "expert_gemm_ref",
    "silu_mul_ref",
    "e4m3_value",
    "f64_to_e4m3_rne",
    "fp8_block_quant",
    "fp8_dequant",
    "fp8_gemm_ref",
    "k3_kl",
]


# ---------------------------------------------------------------------------
# bf16 storage
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float64.

    bf16 is the upper half of an IEEE float32, so widening the 16 bits to the
    top of a 32-bit word gives the float32 with the same value; float32 widens
    to float64 exactly.
    """
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(x) -> np.ndarray:
    """Accept bf16 bit patterns (uint16) or any real array; return float64."""
    a = np.asarray(x)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


# ---------------------------------------------------------------------------
# Leaf partition and the fixed tree   [IsoExec, Parallelism-invariant kernels]
# ---------------------------------------------------------------------------

def leaf_bounds(K: int, leaves: int) -> list[tuple[int, int]]:
    """Leaf l covers columns ``[l*K/L, (l+1)*K/L)``: contiguous, equal, fixed.

    The count is a power of two (reading R1) and must divide K (reading R2).
    """
    if leaves < 1 or (leaves & (leaves - 1)) != 0:
        raise ValueError("leaves must be a power of two")
    if K % leaves != 0:
        raise ValueError("K must be a multiple of leaves")
    ell = K // leaves
    return [(l * ell, (l + 1) * ell) for l in range(leaves)]


def leaf_tree_f32(partials) -> np.ndarray:
    """Combine float32 leaf partials ``P[0..L-1]`` by the fixed binary tree.

    Reading R1: adjacent leaves are paired level by level,
    ``T(a, b) = T(a, mid) + T(mid, b)`` with ``mid = (a + b) / 2``, every add a
    float32 add rounded to nearest even.  ``partials`` has shape ``[L, ...]``;
    the result has the trailing shape.
    """
    level = [np.asarray(p, dtype=np.float32) for p in partials]
    n = len(level)
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError("leaf count must be a power of two")
    with np.errstate(over="ignore", invalid="ignore"):
        while len(level) > 1:
            level = [np.add(level[2 * i], level[2 * i + 1], dtype=np.float32)
                     for i in range(len(level) // 2)]
    return level[0]


def contraction_ref(A, W, row_chunk: int = 256) -> np.ndarray:
    """Exact contraction ``X[m, n] = sum_k A[m, k] * W[n, k]`` in float64.

    This is the value every leaf schedule approximates [IsoExec,
    Parallelism-invariant kernels].  ``A`` is ``[M, K]`` and ``W`` is ``[N, K]``
    (row-major, K contiguous, the layout of a linear / LM-head weight).  Each
    bf16 x bf16 product is exact in float64; rows are computed in chunks only to
    bound memory (rows are independent, so chunking reorders nothing).
    """
    A64 = as_f64(A)
    W64 = as_f64(W)
    if A64.ndim != 2 or W64.ndim != 2 or A64.shape[1] != W64.shape[1]:
        raise ValueError("A must be [M, K] and W must be [N, K]")
    M = A64.shape[0]
    out = np.empty((M, W64.shape[0]), dtype=np.float64)
    WT = W64.T
    for r0 in range(0, M, row_chunk):
        r1 = min(M, r0 + row_chunk)
        out[r0:r1] = A64[r0:r1] @ WT
    return out


def leaf_tree_gemm_f32(A, W, leaves: int) -> np.ndarray:
    """Float32 model of the leaf-tree contraction.

    Each leaf sum ``P_l[m, n] = sum_{k in leaf l} A[m, k] W[n, k]`` is formed in
    float64 and rounded once to float32; the leaves are then combined by
    ``leaf_tree_f32``.  This equals the GPU bit for bit exactly when every leaf
    sum is representable in float32 and exact in float64 (for example one
    nonzero product per leaf, or small integers); otherwise the rounding inside
    a leaf is not modelled.
    """
    A64 = as_f64(A)
    W64 = as_f64(W)
    K = A64.shape[1]
    parts = []
    for k0, k1 in leaf_bounds(K, leaves):
        parts.append((A64[:, k0:k1] @ W64[:, k0:k1].T).astype(np.float32))
    return leaf_tree_f32(parts)


# ---------------------------------------------------------------------------
# Log-softmax and the sampled-token logprob   [Bit-consistent RL, section 2]
# ---------------------------------------------------------------------------

def lse_ref(X) -> np.ndarray:
    """Row-wise ``log(sum_v exp(X[m, v]))`` in float64, max-shifted (R6)."""
    X = np.asarray(X, dtype=np.float64)
    g = X.max(axis=-1, keepdims=True)
    s = np.exp(X - g).sum(axis=-1, keepdims=True)
    return (g + np.log(s))[..., 0]


def log_softmax_ref(X) -> np.ndarray:
    """Row-wise log-softmax in float64: ``X - lse(X)``."""
    X = np.asarray(X, dtype=np.float64)
    return X - lse_ref(X)[..., None]


def logprob_ref(H, W, ids, row_chunk: int = 256):
    """Logprob of each row's sampled token under ``softmax(H W^T)``.

    Returns ``(logprob[M], lse[M])`` in float64.  ``H`` is ``[M, K]``, ``W`` is
    ``[V, K]``, ``ids`` is ``[M]``.  The logits are never rounded (R5); a row
    whose id lies outside ``[0, V)`` gets NaN (R8).  Rows are processed in
    chunks to bound memory; each row is computed whole (full contraction, then
    max, then sum), so nothing is reordered.
    """
    H64 = as_f64(H)
    W64 = as_f64(W)
    ids = np.asarray(ids, dtype=np.int64)
    M = H64.shape[0]
    V = W64.shape[0]
    if ids.shape != (M,):
        raise ValueError("ids must have shape [M]")
    lp = np.empty(M, dtype=np.float64)
    lse = np.empty(M, dtype=np.float64)
    WT = W64.T
    for r0 in range(0, M, row_chunk):
        r1 = min(M, r0 + row_chunk)
        X = H64[r0:r1] @ WT
        l = lse_ref(X)
        lse[r0:r1] = l
        rid = ids[r0:r1]
        ok = (rid >= 0) & (rid < V)
        picked = np.full(r1 - r0, np.nan)
        rows = np.nonzero(ok)[0]
        picked[rows] = X[rows, rid[rows]]
        lp[r0:r1] = picked - l
    return lp, lse


def gumbel_max_ids(X, G) -> np.ndarray:
    """Sample one id per row from ``softmax(X)`` by the Gumbel-max rule.

    ``G`` holds standard Gumbel noise of the same shape (drawn by the seeded
    input generator); ``argmax(X + G)`` is an exact sample from the softmax.
    Ties go to the lower index (numpy's argmax).
    """
    X = np.asarray(X, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    return np.argmax(X + G, axis=-1).astype(np.int64)


# ---------------------------------------------------------------------------
# MoE-shaped combine   [Bit-consistent RL, sections 4.4 and 4.5]
# ---------------------------------------------------------------------------

def moe_ref(H, W_experts, topk_ids, topk_w, row_chunk: int = 512) -> np.ndarray:
    """``out[t] = sum_s topk_w[t, s] * (H[t] . W_{topk_ids[t, s]}^T)`` in float64.

    ``H`` is ``[T, K]``, ``W_experts`` is ``[E, N, K]``, ``topk_ids`` and
    ``topk_w`` are ``[T, topk]``.  In float64 the order of the expert terms
    changes nothing at the tolerances used.
    """
    H64 = as_f64(H)
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float64)
    T = H64.shape[0]
    E, N, K = np.asarray(W_experts).shape
    out = np.zeros((T, N), dtype=np.float64)
    for e in range(E):
        tok, slot = np.nonzero(ids == e)
        if tok.size == 0:
            continue
        We = as_f64(W_experts[e])
        for r0 in range(0, tok.size, row_chunk):
            t = tok[r0:r0 + row_chunk]
            s = slot[r0:r0 + row_chunk]
            y = H64[t] @ We.T
            np.add.at(out, t, w[t, s][:, None] * y)
    return out


def moe_combine_f32(Y, topk_ids, topk_w) -> np.ndarray:
    """Float32 emulation of the fixed-order expert combine (reading R12).

    ``Y[t, s, :]`` is the float32 output of expert ``topk_ids[t, s]`` for token
    ``t``.  The terms are taken in ascending expert id (equal ids keep their slot
    order), and ``acc = acc + w * y`` is a float32 multiply followed by a
    float32 add, each rounded to nearest even, starting from ``acc = +0``.
    """
    Y = np.asarray(Y, dtype=np.float32)
    ids = np.asarray(topk_ids, dtype=np.int64)
    w = np.asarray(topk_w, dtype=np.float32)
    T, S, N = Y.shape
    out = np.zeros((T, N), dtype=np.float32)
    order = np.argsort(ids, axis=1, kind="stable")
    with np.errstate(over="ignore", invalid="ignore"):
        for j in range(S):
            s = order[:, j]
            rows = np.arange(T)
            term = np.multiply(w[rows, s][:, None], Y[rows, s], dtype=np.float32)
            out = np.add(out, term, dtype=np.float32)
    return out


# ---------------------------------------------------------------------------
# Expert GEMM on two layouts, and the activation between the expert GEMMs
#   [Bit-consistent RL, section 4.4; readings R19, R20]
# ---------------------------------------------------------------------------

def f64_to_bf16_rne(x) -> np.ndarray:
    """Round float64 values to bf16 once, to nearest even; return the uint16 bits.

    bf16 keeps 8 significant bits (exponent range of float32): a normal value
    ``m * 2**e`` with ``m`` in [0.5, 1) rounds to ``rint(m * 2**8) * 2**(e-8)``,
    ``rint`` taking halves to even; below the smallest normal, 2**-126, the
    step is 2**-133.  Values at or past the largest finite bf16 plus half a step
    become infinities.  The rounding is done on the float64 value itself, not
    through float32 (which would round twice).
    """
    v = np.asarray(x, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float64)
    a = np.abs(v)
    nan = np.isnan(v)
    small = a < 2.0 ** -126
    m, e = np.frexp(np.where(small | nan, 1.0, a))
    normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    sub = np.rint(np.where(nan, 0.0, a) * 2.0 ** 133) * 2.0 ** -133
    out = np.where(small, sub, normal)
    top = float(np.ldexp(255.0, 120))          # largest finite bf16: (2 - 2**-7) * 2**127
    out = np.where(out > top, np.inf, out)
    out = np.copysign(out, v)
    bits = (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(nan, np.uint16(0x7FC0), bits).astype(np.uint16)


def expert_row_starts(counts, layout: str, cap: int = 0, align: int = 1):
    """First row of each expert's block (masked) or segment (contiguous).

    Returns ``(starts, rows)``: ``rows[e]`` is the number of expert e's rows the
    layout holds (``min(count, cap)`` when masked).  Contiguous: expert e starts
    at the sum over e' < e of ``count_e'`` rounded up to a multiple of ``align``.
    """
    c = np.maximum(np.asarray(counts, dtype=np.int64), 0)
    if layout == "masked":
        rows = np.minimum(c, cap)
        starts = np.arange(c.size, dtype=np.int64) * cap
    elif layout == "contiguous":
        rows = c
        padded = -(-c // align) * align
        starts = np.concatenate([[0], np.cumsum(padded)[:-1]]).astype(np.int64)
    else:
        raise ValueError(layout)
    return starts, rows


def expert_gemm_ref(X, counts, W_experts, layout: str, cap: int = 0, align: int = 1):
    """Expert GEMM on a layout, fp64: ``Y[r] = X[r] . W_e^T`` for every row r
    the layout gives to expert e; other rows are NaN (not defined)."""
    X64 = as_f64(X)
    starts, rows = expert_row_starts(counts, layout, cap, align)
    E, N, K = np.asarray(W_experts).shape
    Y = np.full((X64.shape[0], N), np.nan)
    for e in range(E):
        if rows[e] == 0:
            continue
        sl = slice(int(starts[e]), int(starts[e] + rows[e]))
        Y[sl] = X64[sl] @ as_f64(W_experts[e]).T
    return Y


def silu_mul_ref(G, U) -> np.ndarray:
    """``bf16(SiLU(g) * u)`` with one rounding (reading R20); uint16 bits.

    ``SiLU(g) = g / (1 + exp(-g))`` in float64 (for g below -700, where
    exp(-g) overflows, g * exp(g), which differs from it by less than float64
    resolves), times u, then ``f64_to_bf16_rne``.
    """
    g = np.asarray(G, dtype=np.float64)
    u = np.asarray(U, dtype=np.float64)
    with np.errstate(over="ignore"):
        silu = np.where(g < -700.0, g * np.exp(np.maximum(g, -745.0)), g / (1.0 + np.exp(-g)))
    return f64_to_bf16_rne(silu * u)


# ---------------------------------------------------------------------------
# Block FP8 (W8A8)   [Bit-consistent RL, sections 4.1 and 4.4; reading R21]
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_value(bits) -> np.ndarray:
    """Value of OCP E4M3 bytes: sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN."""
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    ex, man = (b >> 3) & 0xF, b & 0x7
    mag = np.where(ex == 0, man / 8.0 * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(ex - 7.0))
    return np.where((b & 0x7F) == 0x7F, np.nan, sign * mag)


def f64_to_e4m3_rne(x) -> np.ndarray:
    """Round float64 values with |x| <= 448 to E4M3 once, to nearest even; bytes.

    A normal value keeps 4 significant bits: ``rint(m * 2^4) * 2^(e-4)`` for
    ``x = m * 2^e``, m in [0.5, 1); below the smallest normal, 2^-6, the step
    is 2^-9.  (Values above 448 are outside the block rule and rejected.)
    """
    v = np.asarray(x, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("E4M3 rounding needs finite |x| <= 448")
    m, e = np.frexp(np.where(a == 0, 1.0, a))
    normal = np.ldexp(np.rint(np.ldexp(m, 4)), e - 4)
    r = np.where(a < 2.0 ** -6, np.rint(a * 2.0 ** 9) * 2.0 ** -9, normal)
    # encode: find the byte whose value is r (exact), by field arithmetic
    sub = r < 2.0 ** -6
    code_sub = np.rint(r * 2.0 ** 9).astype(np.int64)                 # 0..8 (8 = smallest normal)
    m2, e2 = np.frexp(np.where(sub | (r == 0), 1.0, r))
    code_norm = ((e2 - 1 + 7) << 3) | (np.rint(m2 * 16).astype(np.int64) - 8)
    code = np.where(sub, code_sub, code_norm)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def _block_exponent(amax) -> np.ndarray:
    """Smallest integer e >= -127 with amax <= 448 * 2^e (0 where amax == 0);
    -127 is the lowest exponent one E8M0 byte holds (and bf16 values never
    need more than 120)."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = ex - 9                                                        # 448 * 2^(ex-9) < 2^ex
    while True:
        low = (a > 0) & (np.ldexp(E4M3_MAX, e) < a)
        if not low.any():
            break
        e = e + low
    while True:
        high = (a > 0) & (np.ldexp(E4M3_MAX, e - 1) >= a)
        if not high.any():
            break
        e = e - high
    return np.where(a > 0, np.maximum(e, -127), 0).astype(np.int64)


def fp8_block_quant(X, block_rows: int, block_cols: int = 128):
    """Block FP8 quantisation of ``X [R, C]`` (reading R21).

    Returns ``(q uint8 [R, C], e int [ceil(R/br), ceil(C/bc)])``: ``e`` the
    block's scale exponent, ``q`` each element times 2^-e rounded to E4M3 once.
    """
    X64 = as_f64(X)
    R, C = X64.shape
    nbr, nbc = -(-R // block_rows), -(-C // block_cols)
    e = np.zeros((nbr, nbc), dtype=np.int64)
    q = np.zeros((R, C), dtype=np.uint8)
    for i in range(nbr):
        for j in range(nbc):
            blk = X64[i * block_rows:(i + 1) * block_rows, j * block_cols:(j + 1) * block_cols]
            ex = int(_block_exponent(np.max(np.abs(blk)) if blk.size else 0.0))
            e[i, j] = ex
            q[i * block_rows:(i + 1) * block_rows, j * block_cols:(j + 1) * block_cols] = \
                f64_to_e4m3_rne(np.ldexp(blk, -ex))
    return q, e


def fp8_dequant(q, e, block_rows: int, block_cols: int = 128) -> np.ndarray:
    """``q * 2^e`` with each element's block exponent, float64 (exact)."""
    v = e4m3_value(q)
    ee = np.repeat(np.repeat(np.asarray(e, dtype=np.int64), block_rows, 0), block_cols, 1)
    return np.ldexp(v, ee[:v.shape[0], :v.shape[1]])


def fp8_gemm_ref(qa, ea, qw, ew, row_chunk: int = 256) -> np.ndarray:
    """W8A8 block-FP8 GEMM in float64: ``dequant(A) dequant(W)^T`` with A in
    1 x 128 blocks and W in 128 x 128 blocks."""
    A = fp8_dequant(qa, ea, 1)
    W = fp8_dequant(qw, ew, 128)
    out = np.empty((A.shape[0], W.shape[0]))
    for r0 in range(0, A.shape[0], row_chunk):
        out[r0:r0 + row_chunk] = A[r0:r0 + row_chunk] @ W.T
    return out


# ---------------------------------------------------------------------------
# Router of the MoE layer   [Bit-consistent RL, sections 1 and 4.1; reading R13]
# ---------------------------------------------------------------------------

def route_select(logits, topk: int) -> np.ndarray:
    """Expert ids of the ``topk`` largest logits of each row, largest first.

    Equal logits are taken in ascending expert id (reading R13); +0 and -0 are
    equal; NaN logits come after every other value.  A plain stable sort by the
    key (-logit, expert id).
    """
    X = np.asarray(logits, dtype=np.float64)
    T, E = X.shape
    ids = np.broadcast_to(np.arange(E), X.shape)
    order = np.lexsort((ids, -X), axis=1)   # last key first: -logit, then id
    return order[:, :topk].astype(np.int32)


def route_gates_ref(logits, topk_ids) -> np.ndarray:
    """Softmax over each row's selected logits (fp64): ``exp(l - m) / sum``."""
    X = np.asarray(logits, dtype=np.float64)
    sel = np.take_along_axis(X, np.asarray(topk_ids, dtype=np.int64), axis=1)
    e = np.exp(sel - sel.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def route_ref(H, Wr, topk: int):
    """Router of the MoE layer: (fp64 logits, top-k ids, fp64 gates)."""
    logits = contraction_ref(H, Wr)
    ids = route_select(logits, topk)
    return logits, ids, route_gates_ref(logits, ids)


# ---------------------------------------------------------------------------
# Deterministic Top-K of positions   [Bit-consistent RL, section 4.3]
# ---------------------------------------------------------------------------

def topk_positions(scores, lengths, k: int) -> np.ndarray:
    """Top-``k`` positions of each row by score; ties to the larger position.

    Row r's candidates are its positions ``0 .. lengths[r]-1``.  A position is
    ahead of another when its score is larger, or the scores are equal and its
    position is larger (the 64-bit key of score and in-request position of
    section 4.3); +0 equals -0 and NaN scores come after every number.  The
    ``min(k, lengths[r])`` selected positions are then listed by descending
    position, followed by -1 (invalid) entries up to ``k``.
    """
    S = np.asarray(scores, dtype=np.float64)
    R = S.shape[0]
    out = np.full((R, k), -1, dtype=np.int64)
    for r in range(R):
        n = int(lengths[r])
        s = S[r, :n]
        pos = np.arange(n)
        nan = np.isnan(s)
        key = np.where(nan, 0.0, -s)          # ascending key = descending score
        order = np.lexsort((-pos, key, nan))  # not NaN first, then score, then position
        sel = np.sort(order[:min(k, n)])[::-1]
        out[r, :sel.size] = sel
    return out


# ---------------------------------------------------------------------------
# Harness metric   [Bit-consistent RL, section 3.2: the k3 estimator]
# ---------------------------------------------------------------------------

def k3_kl(logp_a, logp_b) -> float:
    """Mean k3 estimator ``r - 1 - log r`` with ``r = exp(logp_b - logp_a)``."""
    d = np.asarray(logp_b, dtype=np.float64) - np.asarray(logp_a, dtype=np.float64)
    return float(np.mean(np.expm1(d) - d)) if d.size else 0.0
