"""GPU parity of the grouped (MoE expert) GEMM, fp8_grouped_gemm.

Groups are padded with zero rows to multiples of 128 (Ling 2.0 FP8 blog,
"FP8 padding routing map": padded rows do not change the result).  Bar as in
the dense GEMM (1e-3 * R per element, exact zeros where R == 0), plus: every
group equals the dense GEMM with that expert's weights, pad rows are exactly
zero, empty groups are skipped, and rows past the last group are untouched.
Workload: 8192 tokens, hidden 2048, 128 experts of intermediate 768, top-8
Zipf(1.1) routing, gate/up (N=1536, K=2048) and down (N=2048, K=768).
"""
import numpy as np
import pytest
import torch

import fp8_precision_quant_amd as fq
import oracle
import synthetic
from gpu_util import DEV, bf16_parity, gemm_parity, host, to_dev

pytestmark = pytest.mark.gpu

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _codes(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).choice(FINITE, size=shape)


def _scales(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return (np.exp(g.standard_normal(shape)) * 0.01).astype(np.float32)


def _run(a, sa, off, b, sb, out=torch.float32, c=None):
    c = fq.fp8_grouped_gemm(to_dev(a), to_dev(sa), to_dev(off.astype(np.int32)), to_dev(b),
                            to_dev(sb), out_dtype=out, c=c)
    torch.cuda.synchronize()
    return c


def test_small_groups_with_empty_and_ragged():
    counts = [100, 0, 260, 1, 0, 128]
    G, N, K = len(counts), 300, 400
    off = np.concatenate([[0], np.cumsum([-(-c // 128) * 128 for c in counts])])
    M = int(off[-1])
    A = np.zeros((M, K), np.uint8)
    sa = np.zeros((M, 4), np.float32)
    for e, cnt in enumerate(counts):
        A[off[e]:off[e] + cnt] = _codes((cnt, K), 10 + e)
        sa[off[e]:off[e] + cnt] = _scales((cnt, 4), 20 + e)
    B = _codes((G, N, K), 30)
    sb = _scales((G, 3, 4), 31)
    c = host(_run(A, sa, off, B, sb))
    co = oracle.grouped_gemm(A, sa, off, B, sb)
    _, R = oracle.grouped_gemm(A, sa, off, B, sb, f64=True)
    gemm_parity(c, co, R)
    for e, cnt in enumerate(counts):
        assert np.all(c[off[e] + cnt:off[e + 1]] == 0)


def test_rows_past_last_group_untouched():
    G, N, K = 2, 256, 256
    off = np.array([0, 128, 256])
    M_pad = 512                          # last 256 rows belong to no group
    A = _codes((M_pad, K), 40)
    sa = _scales((M_pad, 2), 41)
    B = _codes((G, N, K), 42)
    sb = _scales((G, 2, 2), 43)
    c = torch.full((M_pad, N), -9.0, dtype=torch.float32, device=DEV)
    _run(A, sa, off, B, sb, c=c)
    ch = host(c)
    assert np.all(ch[256:] == -9.0)
    co = oracle.grouped_gemm(A[:256], sa[:256], off, B, sb)
    _, R = oracle.grouped_gemm(A[:256], sa[:256], off, B, sb, f64=True)
    gemm_parity(ch[:256], co, R)


@pytest.fixture(scope="module")
def moe_inputs():
    m = synthetic.moe()
    qa, sa = oracle.quant_1x128(synthetic.bf16_to_f32(m.a_gate_up))
    qa2, sa2 = oracle.quant_1x128(synthetic.bf16_to_f32(m.a_down))
    G = m.w_gate_up.shape[0]
    qgu = np.empty(m.w_gate_up.shape, np.uint8)
    sgu = np.empty((G, 12, 16), np.float32)
    qd = np.empty(m.w_down.shape, np.uint8)
    sd = np.empty((G, 16, 6), np.float32)
    for e in range(G):
        qgu[e], sgu[e] = oracle.quant_128x128(synthetic.bf16_to_f32(m.w_gate_up[e]))
        qd[e], sd[e] = oracle.quant_128x128(synthetic.bf16_to_f32(m.w_down[e]))
    return m, (qa, sa, qgu, sgu), (qa2, sa2, qd, sd)


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_moe_full_size_sampled_rows(moe_inputs, which):
    m, gu, dn = moe_inputs
    qa, sa, qb, sb = gu if which == "gate_up" else dn
    off = m.offsets.astype(np.int64)
    c32 = host(_run(qa, sa, off, qb, sb))
    cb = host(_run(qa, sa, off, qb, sb, out=torch.bfloat16))
    # sample rows from the most and least loaded experts and some pad rows
    big = int(np.argmax(m.counts))
    small = int(np.argmin(m.counts))
    rows = np.concatenate([np.arange(off[big], off[big] + 6), np.arange(off[small], off[small] + 4),
                           synthetic.sample_rows(qa.shape[0], 10, 404)])
    rows = np.unique(rows)
    co = oracle.grouped_gemm(qa, sa, off, qb, sb, rows=rows)
    _, R = oracle.grouped_gemm(qa, sa, off, qb, sb, rows=rows, f64=True)
    gemm_parity(c32[rows], co, R)
    bf16_parity(cb[rows], c32[rows], co, R, oracle.f32_to_bf16_bits(c32[rows]))
    pad = m.token_index < 0
    assert np.all(c32[pad] == 0)
