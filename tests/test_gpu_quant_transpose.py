"""GPU parity of the fused quantize + transpose (fp8_quant_transpose).

Bit-exact against the oracle's definition: the row outputs equal the 1x128
quantization of X and the column outputs equal the 1x128 quantization of
X^T.  Cases: ragged shapes on both axes, fp32 and bf16, one output pair
only, canaries, and the backward workload (dy 4096x14336 with heavy-tailed
outliers, x 4096x4096) at full size.
"""
import numpy as np
import pytest
import torch

import fp8_precision_quant_amd as fq
import oracle
import synthetic
from gpu_util import DEV, assert_canary, host, padded, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _check(xf, xd, rows_out=True, cols_out=True):
    q_row, s_row, q_colT, s_colT = fq.fp8_quant_transpose(xd, rows_out, cols_out)
    torch.cuda.synchronize()
    qr, sr, qc, sc = oracle.quant_transpose(xf)
    if rows_out:
        assert np.array_equal(host(s_row).view(np.uint32), sr.view(np.uint32))
        assert np.array_equal(host(q_row), qr)
    else:
        assert q_row is None
    if cols_out:
        assert np.array_equal(host(s_colT).view(np.uint32), sc.view(np.uint32))
        assert np.array_equal(host(q_colT), qc)
    else:
        assert q_colT is None


@pytest.mark.parametrize("shape", [(1, 1), (5, 300), (128, 128), (130, 257), (300, 200), (640, 384)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged(shape, dtype):
    seed = 40 + shape[0] + 3 * shape[1]
    xf = synthetic.heavy_tail_f32(synthetic.normal_f32(shape, seed, 1e-3), 0.01, seed + 1)
    if dtype == "bf16":
        bits = synthetic.bf16_from_f32(xf)
        _check(synthetic.bf16_to_f32(bits), to_dev_bf16(bits))
    else:
        _check(xf, to_dev(xf))


def test_single_output_pair():
    xf = synthetic.normal_f32((300, 260), 50)
    xd = to_dev(xf)
    _check(xf, xd, rows_out=True, cols_out=False)
    _check(xf, xd, rows_out=False, cols_out=True)


def test_wide_exponent_range_bf16():
    g = np.random.Generator(np.random.PCG64(51))
    xf = (g.standard_normal((512, 384)) * np.exp2(g.integers(-140, 100, size=(512, 1)))
          * np.exp2(g.integers(-30, 0, size=(1, 384)))).astype(np.float32)
    bits = synthetic.bf16_from_f32(xf)
    _check(synthetic.bf16_to_f32(bits), to_dev_bf16(bits))


def test_canaries():
    R, C = 200, 300
    xf = synthetic.normal_f32((R, C), 52)
    xd = to_dev(xf)
    qrb, qr = padded(R, C, 320, torch.uint8, 0x5A)
    srb, sr = padded(R, 3, 4, torch.float32, -3.0)
    qcb, qc = padded(C, R, 208, torch.uint8, 0x5A)
    scb, sc = padded(C, 2, 3, torch.float32, -3.0)
    fq.fp8_quant_transpose(xd, out=(qr, sr, qc, sc))
    torch.cuda.synchronize()
    assert_canary(qrb, R, C, 0x5A)
    assert_canary(srb, R, 3, -3.0)
    assert_canary(qcb, C, R, 0x5A)
    assert_canary(scb, C, 2, -3.0)
    o = oracle.quant_transpose(xf)
    for got, want in zip((qr, sr, qc, sc), o):
        assert np.array_equal(host(got), want)


def test_backward_workload_full_size():
    dy = synthetic.mlp_backward_dy()
    _check(synthetic.bf16_to_f32(dy), to_dev_bf16(dy))
    x, _ = synthetic.mlp_forward(N=128)
    _check(synthetic.bf16_to_f32(x), to_dev_bf16(x))


def test_underflow_monitor_row_vs_transposed():
    """The analog of the pages' underflow monitor (Ling 2.0 FP8 blog): the
    underflow fraction of dy's row tiles and of its transposed tiles, from
    the GPU codes, equals the oracle's."""
    dy = synthetic.mlp_backward_dy(M=1024, N=2048)
    xf = synthetic.bf16_to_f32(dy)
    q_row, _, q_colT, _ = fq.fp8_quant_transpose(to_dev_bf16(dy))
    torch.cuda.synchronize()
    qr, _, qc, _ = oracle.quant_transpose(xf)
    u_row = oracle.underflow_fraction(xf, host(q_row))
    u_col = oracle.underflow_fraction(np.ascontiguousarray(xf.T), host(q_colT))
    assert u_row == oracle.underflow_fraction(xf, qr)
    assert u_col == oracle.underflow_fraction(np.ascontiguousarray(xf.T), qc)
