"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers (numpy PCG64) and lays them out; it holds
none of the quantization or GEMM arithmetic.  Both the GPU library and the CPU
oracle consume the same bytes, so no cross-implementation RNG is needed.

BF16 tensors are returned as ``uint16`` bit patterns (numpy has no bfloat16);
``bf16_to_f32`` widens them exactly.

Workloads (shapes and distributions; the pages give no dataset for this path):

* tiny linear: x, W [256 x 512] fp32 ~N(0,1), 0.1% of entries (distinct,
  seeded positions) multiplied by 100.
* MLP up-projection: x [4096 x 4096] bf16 ~N(0,1); W [14336 x 4096] bf16
  ~N(0, 0.02).
* its backward: dy [4096 x 14336] bf16 ~1e-3 N(0,1), with 0.1% of positions
  multiplied by 10^U(1,3) (heavy tail, sign kept).
* MoE experts: 8192 tokens x hidden 2048, 128 experts, intermediate 768,
  top-8 routing drawn from a Zipf(1.1) popularity (Gumbel-top-k, i.e. sampling
  without replacement), groups padded with zero rows to a multiple of 128.
* long-K: x [16384 x 8192] bf16 with per-row log-normal magnitude,
  x[m,k] = exp(2 u_m) z_mk; W [8192 x 8192] bf16 ~N(0, 0.02).
* optimizer step: fp32 parameters ~N(0, 0.02) (the MLP weight's size by
  default), gradients 1e-3 N(0,1) with the backward's heavy tail, and earlier
  moments m ~ 1e-3 N(0,1), v = (1e-3 z)^2 (fp32 values; each side encodes
  them itself).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ALIGN = 128


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 samples to bf16 (nearest even) -> uint16 bit patterns."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    x = rng(seed).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def normal_bf16(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    return bf16_from_f32(normal_f32(shape, seed, sigma))


def spike_positions(n: int, frac: float, seed: int) -> np.ndarray:
    """round(frac * n) distinct flat positions, seeded."""
    k = int(round(frac * n))
    return rng(seed).permutation(n)[:k]


def with_outliers_f32(x: np.ndarray, frac: float, factor: float, seed: int) -> np.ndarray:
    """Multiply round(frac*size) distinct seeded entries by ``factor``."""
    y = np.array(x, np.float32, copy=True)
    pos = spike_positions(y.size, frac, seed)
    y.reshape(-1)[pos] *= np.float32(factor)
    return y


def heavy_tail_f32(x: np.ndarray, frac: float, seed: int) -> np.ndarray:
    """Multiply round(frac*size) distinct entries by 10^U(1,3) (sign kept)."""
    y = np.array(x, np.float32, copy=True)
    g = rng(seed)
    pos = g.permutation(y.size)[: int(round(frac * y.size))]
    mult = (10.0 ** g.uniform(1.0, 3.0, size=pos.size)).astype(np.float32)
    y.reshape(-1)[pos] *= mult
    return y


def lognormal_rows_f32(shape, seed: int, sigma: float = 2.0) -> np.ndarray:
    """x[m, k] = exp(sigma * u_m) * z_mk with u, z ~ N(0, 1)."""
    g = rng(seed)
    u = g.standard_normal(size=(shape[0], 1), dtype=np.float32)
    z = g.standard_normal(size=shape, dtype=np.float32)
    return (np.exp(np.float32(sigma) * u) * z).astype(np.float32)


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def tiny_linear():
    """x, W: [256 x 512] fp32 ~N(0,1), 0.1% entries x100 (seeds 101, 102)."""
    x = with_outliers_f32(normal_f32((256, 512), 101), 0.001, 100.0, 1101)
    w = with_outliers_f32(normal_f32((256, 512), 102), 0.001, 100.0, 1102)
    return x, w


def mlp_forward(M=4096, N=14336, K=4096):
    """x [M x K] bf16 ~N(0,1) (seed 201), W [N x K] bf16 ~N(0,0.02) (seed 202)."""
    return normal_bf16((M, K), 201), normal_bf16((N, K), 202, 0.02)


def mlp_backward_dy(M=4096, N=14336):
    """dy [M x N] bf16: 1e-3 N(0,1) with 0.1% entries x 10^U(1,3) (seed 301)."""
    dy = heavy_tail_f32(normal_f32((M, N), 301, 1e-3), 0.001, 3301)
    return bf16_from_f32(dy)


@dataclass
class MoEInputs:
    x: np.ndarray             # [T, H] bf16 bits, the token activations
    counts: np.ndarray        # [G] real tokens per expert
    offsets: np.ndarray       # [G+1] int32, padded group starts (multiples of 128)
    token_index: np.ndarray   # [M_pad] token id per gathered row, -1 for pad rows
    a_gate_up: np.ndarray     # [M_pad, H] bf16 bits, gathered (zero pad rows)
    w_gate_up: np.ndarray     # [G, 2*I, H] bf16 bits
    a_down: np.ndarray        # [M_pad, I] bf16 bits (zero pad rows)
    w_down: np.ndarray        # [G, H, I] bf16 bits


def zipf_topk_routing(T: int, G: int, topk: int, s: float, seed: int) -> np.ndarray:
    """[T, topk] distinct expert ids; expert e has popularity (e+1)^-s.

    Gumbel-top-k on log-popularity, which equals sequential sampling without
    replacement.
    """
    g = rng(seed)
    logp = -s * np.log(np.arange(1, G + 1, dtype=np.float64))
    gumbel = -np.log(-np.log(g.uniform(1e-300, 1.0, size=(T, G))))
    keys = logp[None, :] + gumbel
    return np.argsort(-keys, axis=1)[:, :topk]


def moe(T=8192, H=2048, G=128, I=768, topk=8, zipf_s=1.1, with_weights=True):
    x = normal_bf16((T, H), 401)
    choice = zipf_topk_routing(T, G, topk, zipf_s, 402)
    counts = np.bincount(choice.reshape(-1), minlength=G).astype(np.int64)
    padded = -(-counts // ALIGN) * ALIGN
    offsets = np.zeros(G + 1, np.int64)
    offsets[1:] = np.cumsum(padded)
    M_pad = int(offsets[-1])
    token_index = np.full(M_pad, -1, np.int64)
    for e in range(G):
        toks = np.nonzero((choice == e).any(axis=1))[0]   # ascending token ids
        token_index[offsets[e]:offsets[e] + toks.size] = toks
    a = np.zeros((M_pad, H), np.uint16)
    real = token_index >= 0
    a[real] = x[token_index[real]]
    a2 = normal_bf16((M_pad, I), 405)
    a2[~real] = 0
    w_gu = normal_bf16((G, 2 * I, H), 403, 0.02) if with_weights else None
    w_d = normal_bf16((G, H, I), 404, 0.02) if with_weights else None
    return MoEInputs(x, counts, offsets.astype(np.int32), token_index, a, w_gu, a2, w_d)


def moe_backward_dy(m: MoEInputs, seed: int = 406):
    """Output gradients of the two expert GEMMs, gathered like their inputs
    (zero pad rows): dy_gate_up [M_pad, 2I] and dy_down [M_pad, H] bf16 bits,
    1e-3 N(0,1) with 0.1% entries x 10^U(1,3) (the backward recipe)."""
    real = m.token_index >= 0
    M_pad = real.size
    n_gu, n_d = m.w_gate_up.shape[1], m.w_down.shape[1]
    dgu = heavy_tail_f32(normal_f32((M_pad, n_gu), seed, 1e-3), 0.001, seed + 3000)
    dd = heavy_tail_f32(normal_f32((M_pad, n_d), seed + 1, 1e-3), 0.001, seed + 3001)
    dgu[~real] = 0
    dd[~real] = 0
    return bf16_from_f32(dgu), bf16_from_f32(dd)


def long_k(M=16384, N=8192, K=8192):
    """x [M x K] bf16 exp(2u_m) z (seed 501), W [N x K] bf16 ~N(0,0.02) (seed 502)."""
    return bf16_from_f32(lognormal_rows_f32((M, K), 501)), normal_bf16((N, K), 502, 0.02)


def sample_rows(M: int, n: int, seed: int) -> np.ndarray:
    """n distinct sorted row indices of [0, M), seeded."""
    n = min(n, M)
    return np.sort(rng(seed).permutation(M)[:n])


def rows_per_tile(M: int, seed: int, tile: int = 128) -> np.ndarray:
    """One seeded row index inside every tile of `tile` rows of [0, M), sorted."""
    g = rng(seed)
    starts = np.arange(0, M, tile)
    return starts + g.integers(0, np.minimum(tile, M - starts))


def adam_inputs(n=14336 * 4096, seed=601):
    """(p fp32 [n], g fp32 [n], m fp32 [n], v fp32 [n]) for an optimizer step."""
    p = normal_f32((n,), seed, 0.02)
    g = heavy_tail_f32(normal_f32((n,), seed + 1, 1e-3), 0.001, seed + 2)
    m = normal_f32((n,), seed + 3, 1e-3)
    v = np.square(normal_f32((n,), seed + 4, 1e-3))
    return p, g, m, v
