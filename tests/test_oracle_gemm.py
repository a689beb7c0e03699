"""Pins for the oracle's block-scaled GEMM.

The GEMM is the FP8 Linear of the Ling 2.0 FP8 blog ("where does the worry
come from": BF16 Linear -> quantize -> FP8 GEMM) with an FP32 accumulator
("where is error introduced").  What fixes the oracle, other than itself:

* exact rational arithmetic (``fractions.Fraction``) on tiny ragged shapes:
  the oracle's fp32 result lies within the standard dot-product rounding bound
  of the exact value, and its fp64 result within 1e-12 of it;
* a permutation B (one unit code per row): each output is exactly one
  rounded product, which pins the operand roles and the k index;
* unit codes with power-of-two scales that differ per chunk: every output is
  an exactly predictable sum, which pins the chunk-to-scale indexing for the
  forward (row x block), dgrad (KN layout) and wgrad (row x row) modes;
* a numpy fp64 ``matmul`` per chunk (library primitive) at medium size;
* the grouped GEMM equals the per-group dense GEMM, and zero pad rows give 0
  (Ling 2.0 FP8 blog, "FP8 padding routing map": padded rows leave the
  result mathematically unchanged);
* the grouped backward (dgrad with each expert's weight read as stored, and
  wgrad over each group's tokens only) against fp64 ``matmul`` of the
  dequantized operands group by group, and the linearity of wgrad over
  groups (the per-group weight gradients of a split sum to the gradient over
  all tokens).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

U = 2.0 ** -24
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _codes(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).choice(FINITE, size=shape)


def _scales(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return (np.exp(g.standard_normal(shape)) * 0.01).astype(np.float32)


def test_exact_rational_tiny_ragged():
    M, N, K = 3, 5, 300                    # 3 chunks, the last one 44 long
    KB = 3
    A, B = _codes((M, K), 1), _codes((N, K), 2)
    SA, SB = _scales((M, KB), 3), _scales((N, KB), 4)
    C32 = oracle.gemm_f32(A, SA, B, SB)
    C64, R = oracle.gemm_f64(A, SA, B, SB)
    dec = [Fraction(float(v)) for v in oracle.e4m3_decode(np.arange(256, dtype=np.uint8))[:0x7F]]
    decf = {c: (dec[c & 0x7F] if c & 0x80 == 0 else -dec[c & 0x7F]) for c in FINITE.tolist()}
    for m in range(M):
        for n in range(N):
            exact = Fraction(0)
            rsum = Fraction(0)
            for kb in range(KB):
                p = sum((decf[int(A[m, k])] * decf[int(B[n, k])]
                         for k in range(kb * 128, min(K, kb * 128 + 128))), Fraction(0))
                pa = sum((abs(decf[int(A[m, k])] * decf[int(B[n, k])])
                          for k in range(kb * 128, min(K, kb * 128 + 128))), Fraction(0))
                t = Fraction(float(SA[m, kb])) * Fraction(float(SB[n, kb]))
                exact += p * t
                rsum += pa * abs(t)
            assert abs(float(Fraction(float(R[m, n])) - rsum)) <= 1e-12 * float(rsum)
            bound = (127 + 2 + KB) * U * float(rsum) * 1.01
            assert abs(float(Fraction(float(C32[m, n])) - exact)) <= bound
            assert abs(float(Fraction(float(C64[m, n])) - exact)) <= 1e-12 * float(rsum)


def test_permutation_B_pins_operands():
    M, N, K = 40, 300, 300
    A = _codes((M, K), 5)
    SA = _scales((M, 3), 6)
    perm = np.random.Generator(np.random.PCG64(7)).permutation(K)[:N]
    B = np.zeros((N, K), np.uint8)
    B[np.arange(N), perm] = 0x38                      # 1.0
    SB = np.ones((N, 3), np.float32)
    C = oracle.gemm_f32(A, SA, B, SB)
    decA = oracle.e4m3_decode(A)
    expect = decA[:, perm] * SA[:, perm // 128]        # one fp32 rounding each
    # (value equality: a -0 product added to the +0 accumulator gives +0)
    assert np.array_equal(C, expect.astype(np.float32))


def _pow2_case(M, N, K):
    KB = -(-K // 128)
    kb = np.arange(KB)
    lens = np.minimum(128, K - kb * 128).astype(np.float64)
    ea = (kb[None, :] + np.arange(M)[:, None] % 3)              # SA(m,kb) = 2^ea
    eb = (-2 * kb[None, :] + np.arange(N)[:, None] // 128 % 4)  # SB(n,kb) = 2^eb
    expect = np.einsum("k,mk,nk->mn", lens, 2.0 ** ea, 2.0 ** eb)
    return KB, ea, eb, expect


def test_pow2_chunk_scales_forward_row_x_block():
    M, N, K = 6, 384, 520
    KB, ea, eb, expect = _pow2_case(M, N, K)
    A = np.full((M, K), 0x38, np.uint8)
    B = np.full((N, K), 0x38, np.uint8)
    sa = (2.0 ** ea).astype(np.float32)
    sb_block = (2.0 ** eb[::128]).astype(np.float32)            # [ceil(N/128)][KB]
    C = oracle.gemm_blockscaled(A, sa, "row", B, sb_block, "block", "NK")
    assert np.array_equal(C, expect.astype(np.float32))


def test_pow2_chunk_scales_dgrad_KN():
    M, N, K = 5, 256, 384
    KB, ea, eb, expect = _pow2_case(M, N, K)
    A = np.full((M, K), 0x38, np.uint8)
    B_kn = np.full((K, N), 0x38, np.uint8)                      # stored [K][N]
    sa = (2.0 ** ea).astype(np.float32)
    sb_kn = (2.0 ** eb[::128].T).astype(np.float32)              # grid [k-block][n-block]
    C = oracle.gemm_blockscaled(A, sa, "row", B_kn, sb_kn, "block", "KN")
    assert np.array_equal(C, expect.astype(np.float32))


def test_pow2_chunk_scales_wgrad_row_x_row():
    M, N, K = 7, 200, 300
    KB = 3
    g = np.random.Generator(np.random.PCG64(8))
    ea = g.integers(-5, 6, size=(M, KB))
    eb = g.integers(-5, 6, size=(N, KB))
    lens = np.array([128, 128, 44], np.float64)
    expect = np.einsum("k,mk,nk->mn", lens, 2.0 ** ea, 2.0 ** eb)
    A = np.full((M, K), 0x38, np.uint8)
    B = np.full((N, K), 0x38, np.uint8)
    C = oracle.gemm_blockscaled(A, (2.0 ** ea).astype(np.float32), "row",
                                B, (2.0 ** eb).astype(np.float32), "row", "NK")
    assert np.array_equal(C, expect.astype(np.float32))


def test_tensor_scales():
    M, N, K = 9, 130, 260
    A, B = _codes((M, K), 9), _codes((N, K), 10)
    C = oracle.gemm_blockscaled(A, np.float32([[0.5]]), "tensor", B, np.float32([[0.25]]), "tensor")
    ref = oracle.gemm_f32(A, np.full((M, 3), 0.5, np.float32), B, np.full((N, 3), 0.25, np.float32))
    assert np.array_equal(C, ref)


def test_numpy_matmul_reference_medium():
    M, N, K = 64, 256, 640
    KB = 5
    A, B = _codes((M, K), 11), _codes((N, K), 12)
    SA, SB = _scales((M, KB), 13), _scales((N, KB), 14)
    dA = oracle.e4m3_decode(A).astype(np.float64)
    dB = oracle.e4m3_decode(B).astype(np.float64)
    ref = np.zeros((M, N))
    R = np.zeros((M, N))
    for kb in range(KB):
        sl = slice(kb * 128, kb * 128 + 128)
        t = SA[:, kb, None].astype(np.float64) * SB[None, :, kb].astype(np.float64)
        ref += t * (dA[:, sl] @ dB[:, sl].T)
        R += np.abs(t) * (np.abs(dA[:, sl]) @ np.abs(dB[:, sl]).T)
    C32 = oracle.gemm_f32(A, SA, B, SB)
    C64, R64 = oracle.gemm_f64(A, SA, B, SB)
    assert np.all(np.abs(C32 - ref) <= (127 + 2 + KB) * U * R * 1.01)
    assert np.allclose(C64, ref, rtol=0, atol=1e-12 * R.max())
    assert np.allclose(R64, R, rtol=1e-12)


def test_row_subset_matches_full():
    M, N, K = 50, 70, 256
    A, B = _codes((M, K), 15), _codes((N, K), 16)
    SA, SB = _scales((M, 2), 17), _scales((N, 2), 18)
    full = oracle.gemm_f32(A, SA, B, SB)
    rows = np.array([0, 7, 49, 7])
    assert np.array_equal(oracle.gemm_f32(A, SA, B, SB, rows=rows), full[rows])


def test_grouped_equals_per_group_and_pad_rows_zero():
    G, N, K = 3, 256, 384
    counts = [100, 0, 260]
    padded = [-(-c // 128) * 128 for c in counts]
    off = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    M = int(off[-1])
    A = np.zeros((M, K), np.uint8)
    SA = np.zeros((M, 3), np.float32)
    for e in range(G):
        A[off[e]:off[e] + counts[e]] = _codes((counts[e], K), 20 + e)
        SA[off[e]:off[e] + counts[e]] = _scales((counts[e], 3), 30 + e)
    B = np.stack([_codes((N, K), 40 + e) for e in range(G)])
    SB = np.stack([_scales((2, 3), 50 + e) for e in range(G)])
    C = oracle.grouped_gemm(A, SA, off, B, SB)
    for e in range(G):
        lo = int(off[e])
        real = slice(lo, lo + counts[e])
        ref = oracle.gemm_blockscaled(A[real], SA[real], "row", B[e], SB[e], "block")
        assert np.array_equal(C[real], ref)
        pad = slice(lo + counts[e], int(off[e + 1]))
        assert np.all(C[pad] == 0)


def test_bf16_output_rounding_matches_torch():
    g = np.random.Generator(np.random.PCG64(21))
    x = (g.standard_normal(1 << 16) * 10.0 ** g.uniform(-30, 30, 1 << 16)).astype(np.float32)
    ties = (np.arange(1 << 12, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16_bits(x), ref)


def _dequant_rows(codes, scales):
    """fp64 values of 1x128-tiled codes (exact)."""
    d = oracle.e4m3_decode(codes).astype(np.float64)
    return d * np.repeat(scales.astype(np.float64), 128, axis=1)[:, :d.shape[1]]


def _dequant_blocks(codes, scales):
    d = oracle.e4m3_decode(codes).astype(np.float64)
    s = np.repeat(np.repeat(scales.astype(np.float64), 128, axis=0), 128, axis=1)
    return d * s[:d.shape[0], :d.shape[1]]


def _groups(counts):
    padded = [-(-c // 128) * 128 for c in counts]
    return np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)


def test_grouped_dgrad_against_dequantized_matmul():
    # dX[rows of e] = dY[rows of e] @ W_e with W_e's blocks as stored: a
    # transposed block grid or a swapped operand shows up as a large error
    G, N, K = 3, 384, 200
    counts = [130, 0, 100]
    off = _groups(counts)
    M = int(off[-1])
    A = np.zeros((M, N), np.uint8)
    SA = np.zeros((M, 3), np.float32)
    for e in range(G):
        A[off[e]:off[e] + counts[e]] = _codes((counts[e], N), 60 + e)
        SA[off[e]:off[e] + counts[e]] = _scales((counts[e], 3), 70 + e)
    W = np.stack([_codes((N, K), 80 + e) for e in range(G)])
    SW = np.stack([_scales((3, 2), 90 + e) for e in range(G)])
    C32 = oracle.grouped_gemm_dgrad(A, SA, off, W, SW)
    C64, R = oracle.grouped_gemm_dgrad(A, SA, off, W, SW, f64=True)
    for e in range(G):
        rows = slice(int(off[e]), int(off[e + 1]))
        if counts[e] == 0:
            continue
        ref = _dequant_rows(A[rows], SA[rows]) @ _dequant_blocks(W[e], SW[e])
        assert np.allclose(C64[rows], ref, rtol=0, atol=1e-12 * max(R[rows].max(), 1e-30))
        assert np.all(np.abs(C32[rows] - ref) <= (127 + 2 + 3) * U * R[rows] * 1.01)
    assert np.all(C32[off[0] + counts[0]:off[1]] == 0)


def test_grouped_wgrad_per_group_and_linearity():
    # dW_e = dY^T[:, tokens of e] @ X[tokens of e]; an empty group is 0; the
    # per-group gradients add up to the gradient over all tokens
    G, N, K = 4, 150, 260
    counts = [200, 0, 128, 60]
    off = _groups(counts)
    M = int(off[-1])
    g = np.random.Generator(np.random.PCG64(7))
    dy = g.standard_normal((M, N)).astype(np.float32)
    x = g.standard_normal((M, K)).astype(np.float32)
    for e in range(G):                       # pad rows are zero
        dy[off[e] + counts[e]:off[e + 1]] = 0
        x[off[e] + counts[e]:off[e + 1]] = 0
    at, sat = oracle.quant_1x128(np.ascontiguousarray(dy.T))
    bt, sbt = oracle.quant_1x128(np.ascontiguousarray(x.T))
    C32 = oracle.grouped_gemm_wgrad(at, sat, bt, sbt, off)
    C64, R = oracle.grouped_gemm_wgrad(at, sat, bt, sbt, off, f64=True)
    da, db = _dequant_rows(at, sat), _dequant_rows(bt, sbt)
    for e in range(G):
        tok = slice(int(off[e]), int(off[e + 1]))
        ref = da[:, tok] @ db[:, tok].T
        if counts[e] == 0:
            assert np.all(C32[e] == 0) and np.all(C64[e] == 0)
            continue
        assert np.allclose(C64[e], ref, rtol=0, atol=1e-12 * R[e].max())
        kb = (int(off[e + 1]) - int(off[e])) // 128
        assert np.all(np.abs(C32[e] - ref) <= (127 + 2 + kb) * U * R[e] * 1.01)
    whole = da @ db.T
    assert np.allclose(C64.sum(axis=0), whole, rtol=0, atol=1e-12 * R.sum(axis=0).max())
    rows = np.array([3, 0, 149])
    assert np.array_equal(oracle.grouped_gemm_wgrad(at, sat, bt, sbt, off, rows=rows), C32[:, rows])
