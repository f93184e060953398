"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module produces inputs only: bf16 activations and weights, sampled-token
ids, Gumbel noise, MoE routings and the row orders of the prefill / decode
splits.  It holds none of the method's arithmetic (no contraction, no tree, no
softmax over the vocabulary) and imports neither the oracle nor the product
library.

Recipe (each config has a fixed seed; children of ``SeedSequence(seed)`` feed
the separate streams, so changing one stream never shifts another):

* values: float32 draws from ``numpy.random.Generator(PCG64)``; activations
  N(0, 1), weights N(0, 0.02) (the scaling multiply is float32), rounded to
  bf16 by round-to-nearest-even on the bit pattern;
* ids: uniform in ``[0, V)`` where a config says so; where ids must be drawn
  from the softmax itself, this module supplies the Gumbel noise and the caller
  takes the argmax with reference logits;
* prefill / decode: ``n_seq`` sequences of ``n_pos`` positions; the prefill
  chunk is sequence-major, decode step ``t`` holds position ``t`` of every
  sequence (shuffled with a seeded permutation where a config asks for mixed
  sequence origins);
* MoE routing inputs for the expert combine: ``topk`` distinct experts per
  token drawn uniformly and flat-Dirichlet gate weights (float32); no router
  arithmetic (the router is a separate entry point checked against the
  oracle);
* indexer scores for the Top-K of positions: float32 N(0, 1) draws, by default
  rounded to bf16 values so that equal scores are common; request lengths
  uniform in a stated range.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "normal_bf16",
    "Config",
    "CONFIGS",
    "streams",
    "uniform_ids",
    "gumbel",
    "routing_input",
    "prefill_decode_rows",
    "integer_bf16",
    "indexer_scores",
    "request_lengths",
]


def _round_bf16_into(x: np.ndarray, out: np.ndarray, tmp: np.ndarray) -> None:
    """bf16 bits of float32 ``x`` into ``out`` (uint16), using ``tmp`` (uint32) as scratch."""
    u = x.view(np.uint32)
    np.right_shift(u, np.uint32(16), out=tmp)
    np.bitwise_and(tmp, np.uint32(1), out=tmp)
    np.add(tmp, np.uint32(0x7FFF), out=tmp)
    np.add(tmp, u, out=tmp)
    np.right_shift(tmp, np.uint32(16), out=tmp)
    np.copyto(out, tmp, casting="unsafe")


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Finite inputs only.  Adding ``0x7FFF`` plus the lowest kept bit to the
    32-bit pattern and keeping the upper 16 bits rounds the dropped half to
    nearest with ties to even.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _round_bf16_into(x.reshape(-1), out.reshape(-1), np.empty(x.size, dtype=np.uint32))
    return out


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0,
                chunk: int = 1 << 22) -> np.ndarray:
    """N(0, std) draws as bf16 bit patterns (uint16).

    float32 standard normals are drawn in order, scaled by ``std`` in float32
    and rounded to bf16; the chunking only bounds memory (the stream is consumed
    identically for any chunk size).
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    buf = np.empty(min(chunk, max(n, 1)), dtype=np.float32)
    tmp = np.empty(buf.size, dtype=np.uint32)
    s = np.float32(std)
    for i in range(0, n, chunk):
        j = min(n, i + chunk)
        x = buf[: j - i]
        rng.standard_normal(out=x, dtype=np.float32)
        if std != 1.0:
            np.multiply(x, s, out=x)
        _round_bf16_into(x, out[i:j], tmp[: j - i])
    return out.reshape(shape)


def integer_bf16(rng: np.random.Generator, shape, lo: int, hi: int) -> np.ndarray:
    """Uniform integers in ``[lo, hi]`` as bf16 bit patterns (exact for |v| <= 256)."""
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(v)


def sign_bf16(rng: np.random.Generator, shape, exp2: int = 0, chunk: int = 1 << 24) -> np.ndarray:
    """Uniform random signs times ``2**exp2`` as bf16 bit patterns (uint16).

    Element i takes its sign from bit i (least significant first) of the raw
    64-bit outputs of ``rng``'s bit generator, so the values do not depend on
    the chunk size, which only bounds memory (rounded up to a multiple of 64).
    """
    if not -126 <= exp2 <= 127:
        raise ValueError("exp2 must give a normal bf16 power of two")
    n = int(np.prod(shape))
    chunk = -(-max(int(chunk), 64) // 64) * 64
    out = np.empty(n, dtype=np.uint16)
    mag = np.uint16((exp2 + 127) << 7)
    for i in range(0, n, chunk):
        j = min(n, i + chunk)
        words = rng.bit_generator.random_raw(-(-(j - i) // 64)).astype("<u8")
        bits = np.unpackbits(words.view(np.uint8), bitorder="little")[:j - i]
        out[i:j] = bits.astype(np.uint16) << 15
        out[i:j] |= mag
    return out.reshape(shape)


@dataclass(frozen=True)
class Config:
    """One workload: sizes, leaf count and seed."""
    name: str
    K: int
    N: int          # output columns (vocabulary size for the LM-head configs)
    leaves: int
    seed: int
    M: tuple = ()   # row counts exercised
    n_seq: int = 0  # prefill / decode split
    n_pos: int = 0
    experts: int = 0
    topk: int = 0
    tokens: int = 0


CONFIGS = {
    # Tiny: hidden 512, vocab 4096, 1..64 rows, uniform ids.
    "tiny": Config("tiny", K=512, N=4096, leaves=8, seed=1000,
                   M=tuple(range(1, 65))),
    # Linear layer 4096 x 4096 with the row counts that straddle tile edges.
    "linear": Config("linear", K=4096, N=4096, leaves=8, seed=1001,
                     M=(1, 7, 64, 512, 4096, 4097)),
    # LM head: hidden 4096, vocab 151936; 8192 tokens = 128 sequences x 64.
    "lmhead": Config("lmhead", K=4096, N=151936, leaves=8, seed=1002,
                     M=(8192,), n_seq=128, n_pos=64),
    # MoE-shaped: 64 experts of 2048 -> 1408, top-8 of 4096 tokens.
    "moe": Config("moe", K=2048, N=1408, leaves=8, seed=1003,
                  experts=64, topk=8, tokens=4096),
    # Large: hidden 7168, vocab 129280, 16 leaves; 16384 = 256 sequences x 64.
    "large": Config("large", K=7168, N=129280, leaves=16, seed=1004,
                    M=(16384,), n_seq=256, n_pos=64),
    # Sparse-attention indexer Top-K: 128 query rows over histories of up to
    # 65536 positions (N = row pitch), k = 2048 selected per row.
    "indexer": Config("indexer", K=0, N=65536, leaves=0, seed=1005,
                      topk=2048, tokens=128),
}

# Appending keeps every existing stream (child i of the seed sequence is fixed by i).
_STREAMS = ("H", "W", "ids", "perm", "route", "gumbel", "extra", "router", "scores", "lengths")


def streams(seed: int) -> dict:
    """Independent generators for one config, keyed by purpose."""
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {k: np.random.Generator(np.random.PCG64(c)) for k, c in zip(_STREAMS, children)}


def uniform_ids(rng: np.random.Generator, M: int, V: int) -> np.ndarray:
    """Sampled-token ids uniform in ``[0, V)``, int64."""
    return rng.integers(0, V, size=M, dtype=np.int64)


def gumbel(rng: np.random.Generator, shape) -> np.ndarray:
    """Standard Gumbel noise ``-log(-log U)``, U uniform in (0, 1), float64."""
    u = rng.random(shape)
    u = np.clip(u, np.finfo(np.float64).tiny, 1.0 - np.finfo(np.float64).epsneg)
    return -np.log(-np.log(u))


def routing_input(rng: np.random.Generator, T: int, E: int, topk: int):
    """MoE routing input: ``(topk_ids int32 [T, topk], topk_w float32 [T, topk])``.

    A plain sample with the structure of a top-k routing, not a router: each
    token gets ``topk`` distinct experts drawn uniformly (the first ``topk`` of a
    random permutation of the experts), and gate weights drawn from the flat
    Dirichlet distribution (independent unit exponentials divided by their
    sum: positive, summing to 1), stored as float32.  The router itself (top-k
    of the router logits and a softmax over them) is the GPU path's
    ``tig_moe_route`` and the oracle's routing functions, not this module.
    """
    ids = np.argsort(rng.random((T, E)), axis=1, kind="stable")[:, :topk]
    g = rng.exponential(size=(T, topk))
    w = g / g.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


def prefill_decode_rows(n_seq: int, n_pos: int, rng: np.random.Generator | None = None):
    """Row orders for one prefill chunk and for ``n_pos`` decode steps.

    Row ``r = s * n_pos + t`` is position ``t`` of sequence ``s``; the prefill
    chunk holds every row in that sequence-major order.  Decode step ``t`` holds
    position ``t`` of every sequence; with ``rng`` the sequences of each step are
    put in a fresh seeded order (mixed sequence origins).  Returns
    ``(prefill_rows [n_seq*n_pos], decode_steps [n_pos, n_seq])`` as int64.
    """
    prefill = np.arange(n_seq * n_pos, dtype=np.int64)
    steps = np.empty((n_pos, n_seq), dtype=np.int64)
    for t in range(n_pos):
        seqs = np.arange(n_seq) if rng is None else rng.permutation(n_seq)
        steps[t] = seqs * n_pos + t
    return prefill, steps


def indexer_scores(rng: np.random.Generator, R: int, n: int, grid: str = "bf16") -> np.ndarray:
    """Indexer scores, float32 ``[R, n]``, from N(0, 1) draws.

    ``grid="bf16"``: rounded to bf16 values (a few thousand distinct values per
    row, so equal scores are common); ``"int"``: integers in ``[-4, 4]`` (ties
    everywhere); ``"f32"``: the float32 draws as they are.
    """
    if grid == "int":
        return rng.integers(-4, 5, size=(R, n)).astype(np.float32)
    v = rng.standard_normal((R, n), dtype=np.float32)
    if grid == "f32":
        return v
    if grid != "bf16":
        raise ValueError(grid)
    return (f32_to_bf16_bits(v).astype(np.uint32) << 16).view(np.float32)


def request_lengths(rng: np.random.Generator, R: int, lo: int, hi: int) -> np.ndarray:
    """Per-row history lengths, int32, uniform in ``[lo, hi]``."""
    return rng.integers(lo, hi + 1, size=R).astype(np.int32)
