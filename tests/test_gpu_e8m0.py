"""GPU parity of the power-of-two (E8M0) scale path: fp8_quant_blockwise_e8m0,
fp8_quant_transpose_e8m0 and fp8_gemm_e8m0, against the oracle.

Bars: quantization bit-exact (codes and scale bytes); GEMM within
1e-3 * R per element (R = sum of |products| times the scales, from the
oracle's fp64 pass) on the decoded scales, exact where every partial sum is
representable (unit codes, a permutation operand).  Cases: every finite bf16
pattern, tiles across the whole exponent range (zero, subnormal, huge),
ragged shapes, fp32 and bf16 inputs, all three GEMM layouts, K = 0 and
canaries, the MLP workload at full size on sampled rows, and the long-K
workload comparing power-of-two, fp32 block and per-tensor scales.
"""
import numpy as np
import pytest
import torch

import fp8_precision_quant_amd as fq
import oracle
import synthetic
from gpu_util import DEV, assert_canary, bf16_parity, gemm_parity, host, padded, to_dev, to_dev_bf16
from test_gpu_quant import _wide_range_bf16

pytestmark = pytest.mark.gpu

KIND = {"row": fq.ROW_1x128, "block": fq.BLOCK_128x128}
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _orc_quant(x, kind):
    return oracle.quant_1x128_pow2(x) if kind == "row" else oracle.quant_128x128_pow2(x)


def _check_quant(x_f32, x_dev, kind):
    q, e = fq.fp8_quant_blockwise_e8m0(x_dev, KIND[kind])
    torch.cuda.synchronize()
    q, e = host(q), host(e)
    qo, eo = _orc_quant(x_f32, kind)
    bad = np.argwhere(e != eo)
    assert bad.size == 0, "scale bytes differ at %s (gpu %s, oracle %s)" % (
        bad[:5].tolist(), e[tuple(bad[0])], eo[tuple(bad[0])])
    bad = np.argwhere(q != qo)
    assert bad.size == 0, "codes differ at %s (gpu %s, oracle %s)" % (
        bad[:5].tolist(), q[tuple(bad[0])], qo[tuple(bad[0])])
    assert e.min() >= 1 and e.max() <= 247


@pytest.mark.parametrize("kind", ["row", "block"])
def test_all_bf16_patterns(kind):
    g = np.random.Generator(np.random.PCG64(21))
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allb[(allb & 0x7F80) != 0x7F80]
    bits = g.permutation(finite)
    bits = np.concatenate([bits, np.zeros(-bits.size % 512, np.uint16)]).reshape(-1, 512)
    _check_quant(synthetic.bf16_to_f32(bits), to_dev_bf16(bits), kind)


@pytest.mark.parametrize("kind", ["row", "block"])
def test_wide_exponent_range(kind):
    bits = _wide_range_bf16(1024, 640, 22)
    _check_quant(synthetic.bf16_to_f32(bits), to_dev_bf16(bits), kind)


@pytest.mark.parametrize("shape", [(1, 1), (3, 130), (129, 257), (300, 1000)])
@pytest.mark.parametrize("kind", ["row", "block"])
def test_fp32_ragged_and_special_tiles(shape, kind):
    R, C = shape
    g = np.random.Generator(np.random.PCG64(R * 7 + C))
    x = (g.standard_normal((R, C)) * 10.0 ** g.uniform(-30, 30, (R, 1))).astype(np.float32)
    if C > 128:
        x[:, :128] = 0.0                                   # zero tiles: e = -126
        x[0, 128:] = np.float32(1e-44)                     # subnormal amax
    if R > 2:
        x[1, :] = np.float32(448.0 * 2.0 ** int(g.integers(-20, 20)))   # amax = 448 2^j exactly
        x[2, :] = -np.nextafter(np.float32(448.0 * 2.0 ** 3), np.float32(np.inf))   # one ulp above
    _check_quant(x, to_dev(x), kind)


@pytest.mark.parametrize("shape", [(1, 1), (130, 260), (256, 384), (200, 129)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quant_transpose_parity(shape, dtype):
    R, C = shape
    if dtype == "bf16":
        bits = _wide_range_bf16(R, C, R + C)
        x, xd = synthetic.bf16_to_f32(bits), to_dev_bf16(bits)
    else:
        x = synthetic.lognormal_rows_f32((R, C), R * 3 + C)
        xd = to_dev(x)
    q_row, e_row, q_colT, e_colT = fq.fp8_quant_transpose_e8m0(xd)
    torch.cuda.synchronize()
    o = oracle.quant_transpose_pow2(x)
    for got, want in zip((q_row, e_row, q_colT, e_colT), o):
        assert np.array_equal(host(got), want)


def test_quant_canaries():
    R, C = 130, 300
    x = synthetic.normal_f32((R, C), 31)
    qbuf, q = padded(R, C, 320, torch.uint8, 0x5A)
    ebuf, e = padded(R, 3, 8, torch.uint8, 0xA5)
    fq.fp8_quant_blockwise_e8m0(to_dev(x), fq.ROW_1x128, q=q, e=e)
    torch.cuda.synchronize()
    assert_canary(qbuf, R, C, 0x5A)
    assert_canary(ebuf, R, 3, 0xA5)
    qo, eo = oracle.quant_1x128_pow2(x)
    assert np.array_equal(host(q), qo) and np.array_equal(host(e), eo)


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------

def _codes(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).choice(FINITE, size=shape)


def _ebytes(shape, seed, lo=117, hi=128):
    return np.random.Generator(np.random.PCG64(seed)).integers(lo, hi, size=shape).astype(np.uint8)


def _eb_shape(kind, layout, N, K):
    KB, NB = -(-K // 128), -(-N // 128)
    if kind == "row":
        return (N, KB)
    return (NB, KB) if layout == "NK" else (KB, NB)


LAYOUT = {"NK": fq.B_NK, "KN": fq.B_KN}


def _run(a, ea, b, eb, kind, layout, out=torch.float32):
    c = fq.fp8_gemm_e8m0(to_dev(a), to_dev(ea), to_dev(b), to_dev(eb), KIND[kind], LAYOUT[layout],
                         out_dtype=out)
    torch.cuda.synchronize()
    return host(c)


def _oracle(a, ea, b, eb, kind, layout, rows=None):
    sa, sb = oracle.e8m0_decode(ea), oracle.e8m0_decode(eb)
    co = oracle.gemm_blockscaled(a, sa, "row", b, sb, kind, layout, rows=rows)
    _, R = oracle.gemm_blockscaled(a, sa, "row", b, sb, kind, layout, rows=rows, f64=True)
    return co, R


def _parity(a, ea, b, eb, kind, layout, rows=None, bf16=True):
    c = _run(a, ea, b, eb, kind, layout)
    co, R = _oracle(a, ea, b, eb, kind, layout, rows)
    sel = slice(None) if rows is None else rows
    worst = gemm_parity(c[sel], co, R)
    if bf16:
        cb = _run(a, ea, b, eb, kind, layout, out=torch.bfloat16)
        bf16_parity(cb[sel], c[sel], co, R, oracle.f32_to_bf16_bits(c[sel]))
    return worst


def test_permutation_operand_pins_scale_lanes():
    # B selects one column of A per output column: C[m][n] is one product,
    # dec(A[m][perm n]) * 2^(ea - 127) * 2^(eb - 127), exact -- a scale byte
    # applied to the wrong row, column or chunk changes it
    M, N, K = 64, 384, 384
    A = _codes((M, K), 41)
    ea = _ebytes((M, 3), 42)
    perm = np.random.Generator(np.random.PCG64(43)).permutation(K)[:N]
    B = np.zeros((N, K), np.uint8)
    B[np.arange(N), perm] = 0x38
    dec = oracle.e4m3_decode(A).astype(np.float64)
    sa = 2.0 ** (ea.astype(np.int64) - 127)
    for kind, layout in [("block", "NK"), ("block", "KN"), ("row", "NK")]:
        eb = _ebytes(_eb_shape(kind, layout, N, K), 44)
        sb = 2.0 ** (eb.astype(np.int64) - 127)
        if kind == "row":
            sbn = sb[np.arange(N), perm // 128]
        elif layout == "NK":
            sbn = sb[np.arange(N) // 128, perm // 128]
        else:
            sbn = sb[perm // 128, np.arange(N) // 128]
        expect = (dec[:, perm] * sa[:, perm // 128] * sbn[None, :]).astype(np.float32)
        bb = B if layout == "NK" else np.ascontiguousarray(B.T)
        c = _run(A, ea, bb, eb, kind, layout)
        assert np.array_equal(c, expect), (kind, layout)


@pytest.mark.parametrize("mode", ["fwd", "dgrad", "wgrad"])
def test_unit_codes_exact(mode):
    # unit codes, scale bytes 124..130: chunk partials 128 (8 in the tail
    # chunk) times 2^[-6, 6]; all partial sums are exact in fp32
    M, N, K = 300, 384, 520
    KB = 5
    A = np.full((M, K), 0x38, np.uint8)
    ea = _ebytes((M, KB), 45, 124, 131)
    if mode == "wgrad":
        eb, B, kind, layout = _ebytes((N, KB), 46, 124, 131), np.full((N, K), 0x38, np.uint8), "row", "NK"
    elif mode == "fwd":
        eb, B, kind, layout = _ebytes((3, KB), 46, 124, 131), np.full((N, K), 0x38, np.uint8), "block", "NK"
    else:
        eb, B, kind, layout = _ebytes((KB, 3), 46, 124, 131), np.full((K, N), 0x38, np.uint8), "block", "KN"
    c = _run(A, ea, B, eb, kind, layout)
    co, _ = _oracle(A, ea, B, eb, kind, layout)
    assert np.array_equal(c, co)


MODES = [("block", "NK"), ("block", "KN"), ("row", "NK")]


@pytest.mark.parametrize("shape", [(1, 1, 1), (300, 200, 300), (256, 256, 512), (64, 1000, 2048),
                                   (513, 129, 129), (17, 700, 4100)])
@pytest.mark.parametrize("modes", MODES)
def test_random_codes_parity(shape, modes):
    M, N, K = shape
    kind, layout = modes
    seed = M * 37 + N * 11 + K
    A = _codes((M, K), seed)
    B = _codes((N, K) if layout == "NK" else (K, N), seed + 1)
    ea = _ebytes((M, -(-K // 128)), seed + 2)
    eb = _ebytes(_eb_shape(kind, layout, N, K), seed + 3)
    _parity(A, ea, B, eb, kind, layout)


@pytest.mark.parametrize("modes", MODES)
def test_matches_the_fp32_scale_path_on_decoded_scales(modes):
    # the same product through fp8_gemm_blockscaled with the decoded scales
    # as fp32: both are within the bar of the oracle, and of each other
    kind, layout = modes
    M, N, K = 512, 768, 1152
    A = _codes((M, K), 51)
    B = _codes((N, K) if layout == "NK" else (K, N), 52)
    ea = _ebytes((M, 9), 53)
    eb = _ebytes(_eb_shape(kind, layout, N, K), 54)
    c2 = _run(A, ea, B, eb, kind, layout)
    c32 = fq.fp8_gemm_blockscaled(to_dev(A), to_dev(oracle.e8m0_decode(ea)), fq.ROW_1x128, to_dev(B),
                                  to_dev(oracle.e8m0_decode(eb)), KIND[kind], LAYOUT[layout],
                                  out_dtype=torch.float32)
    torch.cuda.synchronize()
    _, R = _oracle(A, ea, B, eb, kind, layout)
    gemm_parity(c2, host(c32), R, tol=2e-3)


def test_k_zero_canaries_and_strides():
    a = torch.zeros((5, 16), dtype=torch.uint8, device=DEV)[:, :0]
    b = torch.zeros((7, 16), dtype=torch.uint8, device=DEV)[:, :0]
    e1 = torch.full((5, 4), 127, dtype=torch.uint8, device=DEV)[:, :1]
    e2 = torch.full((1, 4), 127, dtype=torch.uint8, device=DEV)[:, :1]
    c = fq.fp8_gemm_e8m0(a, e1, b, e2, fq.BLOCK_128x128, fq.B_NK, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert c.shape == (5, 7) and np.all(host(c) == 0)
    M, N, K = 130, 200, 384
    A, B = _codes((M, K), 61), _codes((N, K), 62)
    ea, eb = _ebytes((M, 3), 63), _ebytes((2, 3), 64)
    cbuf, c = padded(M, N, 208, torch.float32, -123.0)
    fq.fp8_gemm_e8m0(to_dev(A), to_dev(ea), to_dev(B), to_dev(eb), fq.BLOCK_128x128, fq.B_NK, c=c)
    torch.cuda.synchronize()
    assert_canary(cbuf, M, N, -123.0)
    co, R = _oracle(A, ea, B, eb, "block", "NK")
    gemm_parity(host(c), co, R)


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def test_mlp_step_full_size():
    """MLP up-projection (x [4096x4096], W [14336x4096], dy [4096x14336]) with
    power-of-two scales throughout: the GPU quantizers bit-exact on the whole
    tensors, then forward and dgrad (W as stored) on every output element
    and wgrad (transposed re-quantized operands) on one row of every
    128-row tile."""
    x, w = synthetic.mlp_forward()
    dy = synthetic.mlp_backward_dy()
    xd, wd, dyd = to_dev_bf16(x), to_dev_bf16(w), to_dev_bf16(dy)
    qx, ex, qxT, exT = fq.fp8_quant_transpose_e8m0(xd)
    qw, ew = fq.fp8_quant_blockwise_e8m0(wd, fq.BLOCK_128x128)
    qdy, edy, qdyT, edyT = fq.fp8_quant_transpose_e8m0(dyd)
    torch.cuda.synchronize()
    xf, wf, dyf = synthetic.bf16_to_f32(x), synthetic.bf16_to_f32(w), synthetic.bf16_to_f32(dy)
    o_x = oracle.quant_transpose_pow2(xf)
    o_w = oracle.quant_128x128_pow2(wf)
    o_dy = oracle.quant_transpose_pow2(dyf)
    for got, want in zip((qx, ex, qxT, exT, qw, ew, qdy, edy, qdyT, edyT), o_x + o_w + o_dy):
        assert np.array_equal(host(got), want)
    _parity(o_x[0], o_x[1], o_w[0], o_w[1], "block", "NK")                       # y = x W^T
    _parity(o_dy[0], o_dy[1], o_w[0], o_w[1], "block", "KN", bf16=False)           # dx = dy W
    rows = synthetic.rows_per_tile(14336, 72)
    _parity(o_dy[2], o_dy[3], o_x[2], o_x[3], "row", "NK", rows=rows, bf16=False)     # dW = dy^T x


def _row_error(c, exact):
    """Mean over rows of each output row's relative error: every row counts
    the same, whatever its magnitude (the rows here span four decades)."""
    return float(np.mean(np.linalg.norm(c - exact, axis=1) / np.linalg.norm(exact, axis=1)))


def test_long_k_pow2_vs_fp32_block_vs_tensor(capsys):
    """Long-K stress (x [16384x8192] with log-normal row magnitudes, K =
    8192): parity of the power-of-two path on sampled rows, and how its
    error and underflow sit between the fp32 tile scales and one scale per
    tensor.  A power-of-two scale is at least the fp32 one, so every value
    that underflows with fp32 tile scales underflows with it too; per-tile
    scales of either kind keep the small rows that one tensor scale flushes."""
    x, w = synthetic.long_k()
    xf, wf = synthetic.bf16_to_f32(x), synthetic.bf16_to_f32(w)
    rows = synthetic.sample_rows(xf.shape[0], 12, 504)
    exact = oracle.exact_gemm_f64(xf, wf, rows)
    qx2, ex2 = oracle.quant_1x128_pow2(xf)
    qw2, ew2 = oracle.quant_128x128_pow2(wf)
    _parity(qx2, ex2, qw2, ew2, "block", "NK", rows=rows, bf16=False)
    err, under = {}, {}
    c2, _ = _oracle(qx2, ex2, qw2, ew2, "block", "NK", rows)
    err["pow2"] = _row_error(c2, exact)
    under["pow2"] = oracle.underflow_fraction(xf, qx2)
    for ka, kb in [("row", "block"), ("tensor", "tensor")]:
        qx, sx = oracle.quantize(xf, ka)
        qw, sw = oracle.quantize(wf, kb)
        co = oracle.gemm_blockscaled(qx, sx, ka, qw, sw, kb, "NK", rows=rows)
        err[ka] = _row_error(co, exact)
        under[ka] = oracle.underflow_fraction(xf, qx)
    with capsys.disabled():
        print("\nlong-K mean row relative error %s underflow %s" % (
            {k: "%.3e" % v for k, v in err.items()}, {k: "%.3e" % v for k, v in under.items()}))
    assert under["row"] <= under["pow2"] < under["tensor"]
    assert err["pow2"] < err["tensor"] and err["row"] < err["tensor"]
    assert err["pow2"] <= 1.05 * err["row"]
