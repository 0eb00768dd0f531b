"""Seeded synthetic inputs for the batch-invariant GEMM workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  It is the one piece of code that both the CPU oracle's
tests and the HIP path's tests and benchmark use, so both sides always see the
same bytes.  Everything is generated on the host with numpy's PCG64 generator
(``numpy.random.default_rng(seed)``), fp32 normal draws scaled to the stated
standard deviation; bf16 operands are the fp32 draws rounded to nearest-even
and are returned as ``numpy.uint16`` bit patterns.

Workloads (shapes and distributions follow the router and MoE models named on
the GateLinear and fused-MoE pages; no public dataset is involved):

* ``tiny``     X[M,256], W[32,256], b[32], all N(0,1)/16; probe row 0.
* ``router``   DeepSeek-V4-shaped GateLinear: X[M,4096] ~ N(0,1),
               W[256,4096] ~ N(0,0.02), b[256] ~ N(0,0.01); three probe rows
               planted at several batch positions.
* ``dense_bf16`` X[M,4096], W[4096,4096] ~ N(0,0.02) in bf16.
* ``moe``      Qwen3-30B-A3B-shaped: hidden 2048, 128 experts, intermediate
               768, top-8; X ~ N(0,1) bf16, router W fp32 ~ N(0,0.02),
               expert weights bf16 ~ N(0,0.02).
* ``indexer``  sparse-attention indexer top-k: scores relu(N(0,1)) rounded
               to bf16 precision, [rows, 8192]; decode windows [0, context)
               and packed causal prefill windows.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------- primitives


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal_f32(seed_or_rng, shape, std=1.0) -> np.ndarray:
    g = rng(seed_or_rng) if isinstance(seed_or_rng, (int, np.integer)) else seed_or_rng
    a = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed_or_rng, shape, std=1.0) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(seed_or_rng, shape, std))


def filler_seed(M: int) -> int:
    """Seed of the non-probe rows of a batch of M rows."""
    return 1000 + int(M)


# ------------------------------------------------------------------ batches


@dataclass
class Batch:
    """A batch of M rows with known probe rows planted at known positions."""
    x: np.ndarray                         # [M, K] fp32, or uint16 bf16 bits
    probes: dict = field(default_factory=dict)   # probe id -> list of row positions


def plant(probe_rows: np.ndarray, M: int, positions_of, filler) -> Batch:
    """Filler rows with each probe copied to its positions (later wins)."""
    x = filler.copy()
    probes = {}
    for pid in range(probe_rows.shape[0]):
        pos = sorted({p for p in positions_of(pid) if 0 <= p < M})
        for p in pos:
            x[p] = probe_rows[pid]
        probes[pid] = pos
    # a position claimed by two probes keeps the later one
    for pid in range(probe_rows.shape[0]):
        probes[pid] = [p for p in probes[pid]
                       if all(p not in probes[q] for q in range(pid + 1, probe_rows.shape[0]))]
    return Batch(x=x, probes=probes)


# ------------------------------------------------------------- tiny (fp32)

TINY_N, TINY_K = 32, 256
TINY_M_SWEEP = (1, 8, 15, 16, 17)


@dataclass
class LinearWeights:
    w: np.ndarray          # [N, K] nn.Linear weight (the weight.t() view's memory)
    b: np.ndarray | None   # [N]
    probes: np.ndarray     # [P, K] probe rows


def tiny_weights(seed: int = 0) -> LinearWeights:
    g = rng(seed)
    probe = normal_f32(g, (1, TINY_K), 1.0 / 16.0)
    w = normal_f32(g, (TINY_N, TINY_K), 1.0 / 16.0)
    b = normal_f32(g, (TINY_N,), 1.0 / 16.0)
    return LinearWeights(w=w, b=b, probes=probe)


def tiny_batch(M: int, wts: LinearWeights) -> Batch:
    filler = normal_f32(filler_seed(M), (M, TINY_K), 1.0 / 16.0)
    return plant(wts.probes, M, lambda pid: [0], filler)


# ---------------------------------------------------------- router (fp32)

ROUTER_N, ROUTER_K = 256, 4096
ROUTER_DECODE_M = (1, 2, 4, 8, 15, 16, 17, 32, 33, 64, 128)
ROUTER_PREFILL_M = (1024, 4096)
TILE_STRADDLE = (15, 16, 17, 31, 32, 33)


def router_weights(seed: int = 0, n_probes: int = 3) -> LinearWeights:
    g = rng(seed)
    w = normal_f32(g, (ROUTER_N, ROUTER_K), 0.02)
    b = normal_f32(g, (ROUTER_N,), 0.01)
    probes = normal_f32(g, (n_probes, ROUTER_K), 1.0)
    return LinearWeights(w=w, b=b, probes=probes)


def decode_positions(M: int, pid: int):
    """Probe pid sits at one of {0, M//2, M-1} and at the tile-straddling rows."""
    base = (0, M // 2, M - 1)[pid % 3]
    return [base] + [p for p in TILE_STRADDLE if (p % 3) == pid % 3]


def router_batch(M: int, wts: LinearWeights, copies: int = 0) -> Batch:
    """Decode batches place probes deterministically; with ``copies`` > 0 each
    probe is also planted at that many seeded random positions (prefill)."""
    filler = normal_f32(filler_seed(M), (M, wts.w.shape[1]), 1.0)
    if copies:
        g = rng(7000 + M)
        perm = g.permutation(M)[: copies * wts.probes.shape[0]]
        extra = {pid: list(perm[pid * copies:(pid + 1) * copies]) for pid in range(wts.probes.shape[0])}
        return plant(wts.probes, M, lambda pid: decode_positions(M, pid) + [int(p) for p in extra[pid]], filler)
    return plant(wts.probes, M, lambda pid: decode_positions(M, pid), filler)


# --------------------------------------------------------- dense bf16 GEMM

DENSE_N, DENSE_K = 4096, 4096
DENSE_M_SWEEP = (1, 7, 32, 33, 256, 4096)


def dense_bf16_weights(seed: int = 0, n_probes: int = 3, N=DENSE_N, K=DENSE_K) -> LinearWeights:
    g = rng(seed)
    w = normal_bf16(g, (N, K), 0.02)
    probes = normal_bf16(g, (n_probes, K), 0.02)
    return LinearWeights(w=w, b=None, probes=probes)


def dense_bf16_batch(M: int, wts: LinearWeights) -> Batch:
    filler = normal_bf16(filler_seed(M), (M, wts.w.shape[1]), 0.02)
    return plant(wts.probes, M, lambda pid: decode_positions(M, pid), filler)


# ---------------------------------------------------------------------- MoE

MOE_H, MOE_E, MOE_I, MOE_TOPK = 2048, 128, 768, 8
MOE_M_SWEEP = (1, 16, 64, 256)


@dataclass
class MoEWeights:
    w_router: np.ndarray   # [E, H] fp32
    b_router: np.ndarray | None
    w13: np.ndarray        # [E, 2I, H] bf16 bits: gate rows then up rows
    w2: np.ndarray         # [E, H, I] bf16 bits
    probes: np.ndarray     # [P, H] bf16 bits


def moe_weights(seed: int = 0, H=MOE_H, E=MOE_E, I=MOE_I, n_probes: int = 3) -> MoEWeights:
    g = rng(seed)
    w_router = normal_f32(g, (E, H), 0.02)
    w13 = normal_bf16(g, (E, 2 * I, H), 0.02)
    w2 = normal_bf16(g, (E, H, I), 0.02)
    probes = normal_bf16(g, (n_probes, H), 1.0)
    return MoEWeights(w_router=w_router, b_router=None, w13=w13, w2=w2, probes=probes)


def moe_batch(M: int, wts: MoEWeights) -> Batch:
    filler = normal_bf16(filler_seed(M), (M, wts.w_router.shape[1]), 1.0)
    return plant(wts.probes, M, lambda pid: decode_positions(M, pid), filler)


# ------------------------------------------------------------ indexer top-k

# DeepSeek-V3.2-style sparse-attention indexer (Sparse-MLA page): per query
# row, scores over up to 8192 key columns, top-k in {512, 1024, 2048}.  The
# scores are relu-shaped (relu(q.k) makes exact 0.0 plateaus routine) and
# rounded to bf16 precision, so equal values recur inside a row.
INDEXER_COLS = 8192
INDEXER_TOPK = (512, 1024, 2048)
INDEXER_DECODE_ROWS = (1, 8, 64)
INDEXER_PREFILL_ROWS = 4096


@dataclass
class IndexerBatch:
    scores: np.ndarray          # float32 [rows, cols]
    row_start: np.ndarray       # int64 [rows]
    row_end: np.ndarray         # int64 [rows]


def indexer_scores(seed: int, rows: int, cols: int) -> np.ndarray:
    g = rng(seed)
    s = np.maximum(g.standard_normal((rows, cols), dtype=np.float32), 0.0)
    return bf16_bits_to_f32(f32_to_bf16_bits(s))


def indexer_decode(rows: int, cols: int = INDEXER_COLS, seed: int = 0) -> IndexerBatch:
    """Decode: one row per request, window [0, context length), context
    lengths drawn in [cols/8, cols]; the last row always spans every column."""
    g = rng(5000 + seed + rows)
    re = g.integers(cols // 8, cols + 1, rows).astype(np.int64)
    re[-1] = cols
    return IndexerBatch(indexer_scores(6000 + seed + rows, rows, cols), np.zeros(rows, np.int64), re)


def indexer_prefill(rows: int, cols: int = INDEXER_COLS, seed: int = 0, requests: int = 4) -> IndexerBatch:
    """Prefill: `requests` causal requests packed along both axes.  Request r
    has n_r query rows and a key segment [kv0_r, kv0_r + p_r + n_r) of cached
    prefix p_r plus its own tokens; its query i sees [kv0_r, kv0_r + p_r + i + 1).
    The segments tile [0, cols) (needs cols >= rows)."""
    assert cols >= rows >= requests
    g = rng(7000 + seed + rows)
    n = np.diff([0, *np.sort(g.choice(np.arange(1, rows), requests - 1, replace=False)), rows])
    p = np.diff([0, *np.sort(g.integers(0, cols - rows + 1, requests - 1)), cols - rows])
    ks = np.zeros(rows, np.int64)
    ke = np.zeros(rows, np.int64)
    q0 = kv0 = 0
    for nr, pr in zip(n, p):
        i = np.arange(nr)
        ks[q0:q0 + nr] = kv0
        ke[q0:q0 + nr] = kv0 + pr + i + 1
        q0 += nr
        kv0 += pr + nr
    assert kv0 == cols and q0 == rows
    return IndexerBatch(indexer_scores(8000 + seed + rows, rows, cols), ks, ke)
