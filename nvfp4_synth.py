"""Seeded synthetic inputs shaped like the NVFP4 matmul workloads.

Shared by the tests, the oracle runs and the benchmark.  This module only
draws random numbers (numpy PCG64 via ``default_rng``); it contains none of
the format's arithmetic -- no decoding, scaling or matmul.

Recipe (fixed order inside each workload: words -> scale codes -> global
scales -> activations -> routing):

* packed words: uniform uint32, i.e. uniform random nibbles 0..15;
* E4M3 scale codes: uniform over finite positive codes, 0x01..0x7E for the
  tiny workload and 0x08..0x7E (normal codes, 2^-6 .. 448) elsewhere;
* global scales: float32 log-uniform in [0.5, 2000];
* activations: float32 standard normal (bf16 runs round these to bf16);
* MoE routing: top-k distinct experts per token, uniform without
  replacement.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np

FINITE_POSITIVE_CODES = (0x01, 0x7E)   # every finite positive E4M3 code
NORMAL_POSITIVE_CODES = (0x08, 0x7E)   # 2^-6 .. 448


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def packed_words(g: np.random.Generator, shape) -> np.ndarray:
    return g.integers(0, 2 ** 32, size=shape, dtype=np.uint32)


def scale_codes(g: np.random.Generator, shape, lo_hi=NORMAL_POSITIVE_CODES) -> np.ndarray:
    lo, hi = lo_hi
    return g.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def global_scales(g: np.random.Generator, n: int, lo: float = 0.5, hi: float = 2000.0) -> np.ndarray:
    return np.exp(g.uniform(np.log(lo), np.log(hi), size=n)).astype(np.float32)


def activations(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32)


def routing(g: np.random.Generator, tokens: int, experts: int, top_k: int) -> np.ndarray:
    """[tokens, top_k] int32 distinct expert ids per token."""
    return np.stack([g.permutation(experts)[:top_k] for _ in range(tokens)]).astype(np.int32)


def modelopt_triplet(g: np.random.Generator, batch: int, rows: int, cols: int,
                     with_ws2: bool = True, code_range=NORMAL_POSITIVE_CODES):
    """A ModelOpt-style NVFP4 triplet: weight U8 [batch, rows, cols/2] (two
    nibbles per byte), weight_scale E4M3 codes [batch, rows, cols/16] and
    weight_scale_2 float32 [batch] (log-uniform in [1e-4, 1e-1])."""
    weight = g.integers(0, 256, size=(batch, rows, cols // 2), dtype=np.uint8)
    scale = scale_codes(g, (batch, rows, cols // 16), code_range)
    ws2 = global_scales(g, batch, 1e-4, 1e-1) if with_ws2 else None
    return weight, scale, ws2


@dataclass
class DenseCase:
    """Planes and activations for one dense quantized matmul."""
    M: int
    K: int
    N: int
    transpose: bool
    x: np.ndarray                 # float32 [M, K]
    w: np.ndarray                 # uint32 [N, K/8] (transposed) or [K, N/8]
    scales: np.ndarray            # uint8 w.shape[:-1] + [w.shape[-1]/2]
    gs: Optional[np.ndarray]      # float32 [1] or None


def dense_case(seed: int, M: int, K: int, N: int, transpose: bool = True,
               with_gs: bool = True, code_range=NORMAL_POSITIVE_CODES) -> DenseCase:
    g = rng(seed)
    rows, qlen = (N, K) if transpose else (K, N)
    w = packed_words(g, (rows, qlen // 8))
    sc = scale_codes(g, (rows, qlen // 16), code_range)
    gs = global_scales(g, 1) if with_gs else None
    x = activations(g, (M, K))
    return DenseCase(M, K, N, transpose, x, w, sc, gs)


@dataclass
class BatchedCase:
    """Planes and activations for one batched-weight qmm call."""
    B: int
    XB: int
    M: int
    K: int
    N: int
    transpose: bool
    x: np.ndarray                 # float32 [XB, M, K]
    w: np.ndarray                 # uint32 [B, N, K/8] or [B, K, N/8]
    scales: np.ndarray            # uint8, w.shape[:-1] + [w.shape[-1] / 2]
    gs: Optional[np.ndarray]      # float32 [B] or None


def batched_case(seed: int, B: int, M: int, K: int, N: int, broadcast_x: bool = False,
                 transpose: bool = True, with_gs: bool = True,
                 code_range=NORMAL_POSITIVE_CODES) -> BatchedCase:
    """B weight matrices and either one activation matrix (broadcast_x) or B."""
    g = rng(seed)
    rows, qlen = (N, K) if transpose else (K, N)
    w = packed_words(g, (B, rows, qlen // 8))
    sc = scale_codes(g, (B, rows, qlen // 16), code_range)
    gs = global_scales(g, B) if with_gs else None
    XB = 1 if broadcast_x else B
    x = activations(g, (XB, M, K))
    return BatchedCase(B, XB, M, K, N, transpose, x, w, sc, gs)


@dataclass
class GatherCase:
    """Planes, activations and index pairs for one GatherQMM call."""
    X: int
    M: int
    K: int
    N: int
    E: int
    x: np.ndarray                 # float32 [X, M, K]
    lhs: np.ndarray               # int32 [R]
    rhs: np.ndarray               # int32 [R]
    w: np.ndarray                 # uint32 [E, N, K/8]
    scales: np.ndarray            # uint8 [E, N, K/16]
    gs: Optional[np.ndarray]      # float32 [E] or None
    sorted_indices: bool = False


def gather_case(seed: int, tokens: int, E: int, N: int, K: int, top_k: int,
                sort: bool, with_gs: bool = True, M: int = 1,
                out_of_range: Tuple[int, ...] = ()) -> GatherCase:
    """MoE gather input: each token picks top_k distinct experts; one index
    pair per (token, expert).  sort=True orders the pairs by expert (prefill);
    otherwise they stay in token order (decode).  ``out_of_range`` expert ids
    overwrite evenly spaced pairs after sorting."""
    g = rng(seed)
    w = packed_words(g, (E, N, K // 8))
    sc = scale_codes(g, (E, N, K // 16))
    gs = global_scales(g, E) if with_gs else None
    x = activations(g, (tokens, M, K))
    choice = routing(g, tokens, E, top_k)
    rhs = choice.reshape(-1).astype(np.int32)
    lhs = np.repeat(np.arange(tokens, dtype=np.int32), top_k)
    if sort:
        order = np.argsort(rhs, kind="stable")
        rhs, lhs = rhs[order], lhs[order]
    if out_of_range:
        slots = np.linspace(0, len(rhs) - 1, num=len(out_of_range)).astype(np.int64)
        for s, e in zip(slots, out_of_range):
            rhs[s] = np.int32(e)
    return GatherCase(tokens, M, K, N, E, x, lhs, rhs, w, sc, gs, sort)


# Workloads named by what they are, with their sizes.
WORKLOADS: Dict[str, dict] = {
    "tiny_qmv_m1_k1024_n512_f32": dict(M=1, K=1024, N=512, dtype="f32", gs=False,
                                        codes=FINITE_POSITIVE_CODES, seed=0),
    "decode_qmv_m1_k5376_n21504_bf16": dict(M=1, K=5376, N=21504, dtype="bf16", gs=True,
                                             codes=NORMAL_POSITIVE_CODES, seed=2000),
    "multirow_qmv_k4096_n14336": dict(Ms=(3, 6, 16, 33), K=4096, N=14336, gs=True,
                                      codes=NORMAL_POSITIVE_CODES, seed=3000),
    "prefill_gemm_m2048_k5376_n21504_bf16": dict(M=2048, K=5376, N=21504, dtype="bf16", gs=True,
                                                  codes=NORMAL_POSITIVE_CODES, seed=4000),
    "moe_gather_e128_n1536_k2048_top8": dict(E=128, N=1536, K=2048, top_k=8, sorted_tokens=128,
                                             decode_tokens=(1, 2, 4, 8), seed=5000),
}
