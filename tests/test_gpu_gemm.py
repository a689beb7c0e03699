"""GPU parity of the block-scaled FP8 GEMM (fp8_gemm_blockscaled).

Bar: |C_gpu - C_oracle| <= 1e-3 * R per element, R = sum_kb |SA SB| sum_k
|dec(a) dec(b)| (the dot-product error normalizer: C itself can cancel to
~0); outputs with R == 0 must be exactly 0.  BF16 outputs must be exactly
the GPU's fp32 result rounded to nearest even, and lie within 1e-3 * R plus
half a bf16 ulp of the oracle's fp32 result.  Exactly
representable cases (a permutation operand, unit codes with power-of-two
chunk scales) must match exactly.  Every scale mode and layout is covered:
forward (row x block, B [N][K]), dgrad (row x block, B stored [K][N]),
wgrad (row x row), per-tensor and mixed, ragged shapes on all three axes,
K = 0, canaries, and the workloads' full sizes (whole outputs for the forward
and dgrad, one row in every 128-row tile elsewhere).
"""
import numpy as np
import pytest
import torch

import fp8_precision_quant_amd as fq
import oracle
import synthetic
from gpu_util import (DEV, assert_canary, bf16_parity, gemm_parity, host, padded, to_dev,
                      to_dev_bf16)

pytestmark = pytest.mark.gpu

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
KIND = {"row": fq.ROW_1x128, "block": fq.BLOCK_128x128, "tensor": fq.TENSOR}
LAYOUT = {"NK": fq.B_NK, "KN": fq.B_KN}


def _codes(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).choice(FINITE, size=shape)


def _scales(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return (np.exp(g.standard_normal(shape)) * 0.01).astype(np.float32)


def _b_scale_shape(kind, layout, N, K):
    KB, NB = -(-K // 128), -(-N // 128)
    if kind == "tensor":
        return (1, 1)
    if kind == "row":
        return (N, KB)
    return (NB, KB) if layout == "NK" else (KB, NB)


def _run(a, sa, sa_kind, b, sb, sb_kind, layout, out=torch.float32):
    c = fq.fp8_gemm_blockscaled(to_dev(a), to_dev(sa), KIND[sa_kind], to_dev(b), to_dev(sb),
                                KIND[sb_kind], LAYOUT[layout], out_dtype=out)
    torch.cuda.synchronize()
    return host(c)


def _parity(a, sa, sa_kind, b, sb, sb_kind, layout, rows=None, bf16=True):
    c = _run(a, sa, sa_kind, b, sb, sb_kind, layout)
    co = oracle.gemm_blockscaled(a, sa, sa_kind, b, sb, sb_kind, layout, rows=rows)
    _, R = oracle.gemm_blockscaled(a, sa, sa_kind, b, sb, sb_kind, layout, rows=rows, f64=True)
    sel = slice(None) if rows is None else rows
    worst = gemm_parity(c[sel], co, R)
    if bf16:
        cb = _run(a, sa, sa_kind, b, sb, sb_kind, layout, out=torch.bfloat16)
        bf16_parity(cb[sel], c[sel], co, R, oracle.f32_to_bf16_bits(c[sel]))
    return worst


def test_permutation_operand_pins_mfma_layout():
    M, N, K = 64, 384, 384
    A = _codes((M, K), 1)
    SA = _scales((M, 3), 2)
    perm = np.random.Generator(np.random.PCG64(3)).permutation(K)[:N]
    B = np.zeros((N, K), np.uint8)
    B[np.arange(N), perm] = 0x38                    # 1.0
    expect = (oracle.e4m3_decode(A)[:, perm] * SA[:, perm // 128]).astype(np.float32)
    c = _run(A, SA, "row", B, np.ones((3, 3), np.float32), "block", "NK")
    assert np.array_equal(c, expect)
    c = _run(A, SA, "row", np.ascontiguousarray(B.T), np.ones((3, 3), np.float32), "block", "KN")
    assert np.array_equal(c, expect)
    c = _run(A, SA, "row", B, np.ones((N, 3), np.float32), "row", "NK")
    assert np.array_equal(c, expect)


@pytest.mark.parametrize("mode", ["fwd", "dgrad", "wgrad"])
def test_pow2_chunk_scales_exact(mode):
    # Unit codes: each chunk partial is 128 (8 in the 8-wide tail chunk) times
    # a scale product in [2^-6, 2^6]; every partial sum of the 5 chunks is a
    # multiple of 2^-3 below 2^16, hence exact in fp32 whatever order the
    # chunks are added in.
    M, N, K = 300, 384, 520
    KB = 5
    g = np.random.Generator(np.random.PCG64(4))
    A = np.full((M, K), 0x38, np.uint8)
    ea = g.integers(-3, 4, size=(M, KB))
    sa = (2.0 ** ea).astype(np.float32)
    if mode == "wgrad":
        sb = (2.0 ** g.integers(-3, 4, size=(N, KB))).astype(np.float32)
        B, kind, layout = np.full((N, K), 0x38, np.uint8), "row", "NK"
    elif mode == "fwd":
        sb = (2.0 ** g.integers(-3, 4, size=(3, KB))).astype(np.float32)
        B, kind, layout = np.full((N, K), 0x38, np.uint8), "block", "NK"
    else:
        sb = (2.0 ** g.integers(-3, 4, size=(KB, 3))).astype(np.float32)
        B, kind, layout = np.full((K, N), 0x38, np.uint8), "block", "KN"
    c = _run(A, sa, "row", B, sb, kind, layout)
    co = oracle.gemm_blockscaled(A, sa, "row", B, sb, kind, layout)
    assert np.array_equal(c, co)


MODES = [("row", "block", "NK"), ("row", "block", "KN"), ("row", "row", "NK"),
         ("tensor", "tensor", "NK"), ("row", "tensor", "KN"), ("tensor", "block", "NK"),
         ("tensor", "block", "KN"), ("tensor", "tensor", "KN")]


@pytest.mark.parametrize("shape", [(1, 1, 1), (300, 200, 300), (256, 256, 512), (64, 1000, 2048),
                                   (513, 129, 129), (17, 700, 4100)])
@pytest.mark.parametrize("modes", MODES)
def test_random_codes_parity(shape, modes):
    M, N, K = shape
    sa_kind, sb_kind, layout = modes
    seed = M * 31 + N * 7 + K
    A = _codes((M, K), seed)
    B = _codes((N, K) if layout == "NK" else (K, N), seed + 1)
    sa = _scales((M, -(-K // 128)) if sa_kind == "row" else (1, 1), seed + 2)
    sb = _scales(_b_scale_shape(sb_kind, layout, N, K), seed + 3)
    _parity(A, sa, sa_kind, B, sb, sb_kind, layout)


E4M3_MODES = [("row", "block", "NK"), ("row", "block", "KN"), ("tensor", "tensor", "NK"),
              ("row", "tensor", "KN"), ("tensor", "block", "NK"), ("tensor", "tensor", "KN")]


@pytest.mark.parametrize("shape", [(300, 200, 300), (256, 384, 512), (17, 700, 4100), (513, 129, 129),
                                   (200, 512, 256), (64, 1000, 2048)])
@pytest.mark.parametrize("modes", E4M3_MODES)
def test_e4m3_output_quantizes_the_fp32_result(shape, modes):
    # the stored codes and 1x128 scales are (1) byte for byte the GPU
    # quantizer's output on the same GEMM's fp32 result, and (2) a valid
    # quantization of the oracle's result: each tile's s within the GEMM
    # tolerance of its amax / 448, each dequantized code within half an E4M3
    # step of the oracle's value plus that tolerance
    M, N, K = shape
    sa_kind, sb_kind, layout = modes
    seed = M * 13 + N * 5 + K + 7
    A = _codes((M, K), seed)
    B = _codes((N, K) if layout == "NK" else (K, N), seed + 1)
    sa = _scales((M, -(-K // 128)) if sa_kind == "row" else (1, 1), seed + 2)
    sb = _scales(_b_scale_shape(sb_kind, layout, N, K), seed + 3)
    q, qs = fq.fp8_gemm_blockscaled_e4m3(to_dev(A), to_dev(sa), KIND[sa_kind], to_dev(B), to_dev(sb),
                                         KIND[sb_kind], LAYOUT[layout])
    c = fq.fp8_gemm_blockscaled(to_dev(A), to_dev(sa), KIND[sa_kind], to_dev(B), to_dev(sb),
                                KIND[sb_kind], LAYOUT[layout], out_dtype=torch.float32)
    rq, rs = fq.fp8_quant_blockwise(c, fq.ROW_1x128)
    torch.cuda.synchronize()
    q, qs, rq, rs = host(q), host(qs), host(rq), host(rs)
    assert np.array_equal(q, rq)
    assert np.array_equal(qs.view(np.uint32), rs.view(np.uint32))
    co = oracle.gemm_blockscaled(A, sa, sa_kind, B, sb, sb_kind, layout).astype(np.float64)
    _, R = oracle.gemm_blockscaled(A, sa, sa_kind, B, sb, sb_kind, layout, f64=True)
    NB = -(-N // 128)
    pad = NB * 128 - N
    amax_o = np.abs(np.pad(co, ((0, 0), (0, pad)))).reshape(M, NB, 128).max(axis=2)
    tol_t = 1e-3 * np.pad(R, ((0, 0), (0, pad))).reshape(M, NB, 128).max(axis=2)
    assert np.all(np.abs(qs.astype(np.float64) * 448 - amax_o) <= tol_t * 1.0001 + 1e-30)
    s_full = np.repeat(qs.astype(np.float64), 128, axis=1)[:, :N]
    deq = oracle.e4m3_decode(q).astype(np.float64) * s_full
    half_step = np.maximum(np.abs(co) * 2.0 ** -4, s_full * 2.0 ** -10)
    assert np.all(np.abs(deq - co) <= half_step * 1.0001 + 1e-3 * R * 2 + 1e-30)


def test_k_zero_and_empty():
    a = torch.zeros((5, 16), dtype=torch.uint8, device=DEV)[:, :0]      # K = 0, lda = 16
    b = torch.zeros((7, 16), dtype=torch.uint8, device=DEV)[:, :0]
    c = fq.fp8_gemm_blockscaled(a, to_dev(np.ones((5, 1), np.float32)), fq.ROW_1x128,
                                b, to_dev(np.ones((1, 1), np.float32)), fq.BLOCK_128x128,
                                fq.B_NK, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert c.shape == (5, 7) and np.all(host(c) == 0)
    c = fq.fp8_gemm_blockscaled(torch.empty((0, 128), dtype=torch.uint8, device=DEV),
                                torch.empty((0, 1), dtype=torch.float32, device=DEV), fq.ROW_1x128,
                                to_dev(_codes((8, 128), 5)), to_dev(np.ones((1, 1), np.float32)),
                                fq.BLOCK_128x128, fq.B_NK)
    torch.cuda.synchronize()
    assert c.shape == (0, 8)


def test_output_canaries_and_strides():
    M, N, K = 130, 200, 384
    A, B = _codes((M, K), 6), _codes((N, K), 7)
    sa, sb = _scales((M, 3), 8), _scales((2, 3), 9)
    cbuf, c = padded(M, N, 208, torch.float32, -123.0)
    fq.fp8_gemm_blockscaled(to_dev(A), to_dev(sa), fq.ROW_1x128, to_dev(B), to_dev(sb),
                            fq.BLOCK_128x128, fq.B_NK, c=c)
    torch.cuda.synchronize()
    assert_canary(cbuf, M, N, -123.0)
    co = oracle.gemm_blockscaled(A, sa, "row", B, sb, "block")
    _, R = oracle.gemm_blockscaled(A, sa, "row", B, sb, "block", f64=True)
    gemm_parity(host(c), co, R)


def test_deterministic():
    A, B = _codes((512, 1024), 10), _codes((384, 1024), 11)
    sa, sb = _scales((512, 8), 12), _scales((3, 8), 13)
    c1 = _run(A, sa, "row", B, sb, "block", "NK")
    c2 = _run(A, sa, "row", B, sb, "block", "NK")
    assert np.array_equal(c1, c2)


def test_tiny_linear_forward():
    """x[256x512] W[256x512] fp32 with 0.1% x100 outliers; y = x W^T, fp32 out."""
    x, w = synthetic.tiny_linear()
    qx, sx = fq.fp8_quant_blockwise(to_dev(x), fq.ROW_1x128)
    qw, sw = fq.fp8_quant_blockwise(to_dev(w), fq.BLOCK_128x128)
    y = fq.fp8_gemm_blockscaled(qx, sx, fq.ROW_1x128, qw, sw, fq.BLOCK_128x128, fq.B_NK,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    ox, osx = oracle.quant_1x128(x)
    ow, osw = oracle.quant_128x128(w)
    assert np.array_equal(host(qx), ox) and np.array_equal(host(qw), ow)
    co = oracle.gemm_blockscaled(ox, osx, "row", ow, osw, "block")
    _, R = oracle.gemm_blockscaled(ox, osx, "row", ow, osw, "block", f64=True)
    gemm_parity(host(y), co, R)


def _quantized_mlp():
    x, w = synthetic.mlp_forward()
    qx, sx = oracle.quant_1x128(synthetic.bf16_to_f32(x))
    qw, sw = oracle.quant_128x128(synthetic.bf16_to_f32(w))
    return x, w, qx, sx, qw, sw


def test_mlp_forward_full_size_whole_output():
    """y = x W^T at the forward workload's full size (M = 4096, N = 14336,
    K = 4096, the launch the bench times): every output element, fp32 and
    bf16 (each workgroup walks several tiles here)."""
    x, w, qx, sx, qw, sw = _quantized_mlp()
    _parity(qx, sx, "row", qw, sw, "block", "NK")


def test_e4m3_output_mlp_full_size_sampled_rows():
    """Quantize-on-store at the forward workload's full size (y = x W^T,
    M = 4096, N = 14336, K = 4096, the launch the bench times): codes and
    1x128 scales byte-identical, over the whole output, to the GPU quantizer
    applied to the same GEMM's fp32 output; on sampled rows, a valid
    quantization of the oracle's result (scale within the GEMM tolerance of
    amax / 448, each dequantized code within half an E4M3 step plus it)."""
    x, w, qx, sx, qw, sw = _quantized_mlp()
    A, SA, B, SB = to_dev(qx), to_dev(sx), to_dev(qw), to_dev(sw)
    q, qs = fq.fp8_gemm_blockscaled_e4m3(A, SA, fq.ROW_1x128, B, SB, fq.BLOCK_128x128, fq.B_NK)
    c = fq.fp8_gemm_blockscaled(A, SA, fq.ROW_1x128, B, SB, fq.BLOCK_128x128, fq.B_NK,
                                out_dtype=torch.float32)
    rq, rs = fq.fp8_quant_blockwise(c, fq.ROW_1x128)
    torch.cuda.synchronize()
    assert torch.equal(q, rq)
    assert torch.equal(qs.view(torch.int32), rs.view(torch.int32))
    rows = synthetic.sample_rows(qx.shape[0], 16, 63)
    ridx = torch.from_numpy(rows.astype(np.int64)).to(DEV)
    qh, qsh = host(q.index_select(0, ridx)), host(qs.index_select(0, ridx))
    co = oracle.gemm_blockscaled(qx, sx, "row", qw, sw, "block", "NK", rows=rows).astype(np.float64)
    _, R = oracle.gemm_blockscaled(qx, sx, "row", qw, sw, "block", "NK", rows=rows, f64=True)
    n, N = co.shape
    amax_o = np.abs(co).reshape(n, N // 128, 128).max(axis=2)
    tol_t = 1e-3 * R.reshape(n, N // 128, 128).max(axis=2)
    assert np.all(np.abs(qsh.astype(np.float64) * 448 - amax_o) <= tol_t * 1.0001 + 1e-30)
    s_full = np.repeat(qsh.astype(np.float64), 128, axis=1)
    deq = oracle.e4m3_decode(qh).astype(np.float64) * s_full
    half_step = np.maximum(np.abs(co) * 2.0 ** -4, s_full * 2.0 ** -10)
    assert np.all(np.abs(deq - co) <= half_step * 1.0001 + 1e-3 * R * 2 + 1e-30)


def test_mlp_dgrad_full_size_whole_output():
    """dx = dy W with W read as stored ([N = 14336][K = 4096] is
    [contraction][out]): every output element, fp32 and bf16."""
    x, w, _, _, qw, sw = _quantized_mlp()
    dy = synthetic.mlp_backward_dy()
    q_row, s_row, _, _ = oracle.quant_transpose(synthetic.bf16_to_f32(dy))
    _parity(q_row, s_row, "row", qw, sw, "block", "KN")


def test_mlp_wgrad_full_size_row_per_tile():
    """dW = dy^T x with both operands re-quantized along tokens (14336 x
    4096 output): one seeded row in every 128-row tile, fp32 and bf16."""
    x, _ = synthetic.mlp_forward()
    dy = synthetic.mlp_backward_dy()
    _, _, q_colT, s_colT = oracle.quant_transpose(synthetic.bf16_to_f32(dy))
    _, _, qxT, sxT = oracle.quant_transpose(synthetic.bf16_to_f32(x))
    rows = synthetic.rows_per_tile(q_colT.shape[0], 62)
    _parity(q_colT, s_colT, "row", qxT, sxT, "row", "NK", rows=rows)


def test_long_k_blockwise_vs_tensor_sampled_rows(capsys):
    """Long-K stress (x [16384 x 8192] with log-normal row magnitudes, K =
    8192): parity for both scalings on 256 seeded rows, and the pages' claim
    that fine-grained scaling beats one scale per tensor (less underflow,
    smaller error against the exact product of the bf16 inputs).  The error
    is reported two ways: the Frobenius norm of the sampled block relative to
    the exact one, and the mean over rows of each row's relative error (the
    rows span four decades, so the norm weighs only the largest rows)."""
    x, w = synthetic.long_k()
    xf, wf = synthetic.bf16_to_f32(x), synthetic.bf16_to_f32(w)
    rows = synthetic.sample_rows(xf.shape[0], 256, 503)
    exact = oracle.exact_gemm_f64(xf, wf, rows)
    fro, rowm, under = {}, {}, {}
    for kind_a, kind_b in [("row", "block"), ("tensor", "tensor")]:
        qx, sx = oracle.quantize(xf, kind_a)
        qw, sw = oracle.quantize(wf, kind_b)
        c = _run(qx, sx, kind_a, qw, sw, kind_b, "NK")[rows]
        co = oracle.gemm_blockscaled(qx, sx, kind_a, qw, sw, kind_b, "NK", rows=rows)
        _, R = oracle.gemm_blockscaled(qx, sx, kind_a, qw, sw, kind_b, "NK", rows=rows, f64=True)
        gemm_parity(c, co, R)
        fro[kind_a] = float(np.linalg.norm(co - exact) / np.linalg.norm(exact))
        rowm[kind_a] = float(np.mean(np.linalg.norm(co - exact, axis=1) / np.linalg.norm(exact, axis=1)))
        under[kind_a] = oracle.underflow_fraction(xf, qx)
    with capsys.disabled():
        print("\nlong-K error vs exact (256 rows): Frobenius %s, mean row %s, underflow %s" % (
            {k: "%.4e" % v for k, v in fro.items()}, {k: "%.4e" % v for k, v in rowm.items()},
            {k: "%.3e" % v for k, v in under.items()}))
    assert under["row"] < under["tensor"]
    assert rowm["row"] < rowm["tensor"]
    assert fro["row"] < fro["tensor"]
