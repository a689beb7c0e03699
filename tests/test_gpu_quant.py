"""GPU parity of the tile quantizers (fp8_quant_blockwise) against the oracle.

The bar is bit-exact codes and scale bits.  Cases: every finite bf16 bit
pattern, tiles spanning the whole exponent range (subnormal inputs, subnormal
and zero scales, underflow to signed zero), the exact-code round trip,
ragged shapes on every edge, empty inputs, fp32 inputs, the workloads'
shapes at full size, canary bytes around every output, and run-to-run
determinism.
"""
import numpy as np
import pytest
import torch

import fp8_precision_quant_amd as fq
import oracle
import synthetic
from gpu_util import DEV, assert_canary, host, padded, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

KINDS = {"row": fq.ROW_1x128, "block": fq.BLOCK_128x128, "tensor": fq.TENSOR}


def _gpu_quant(x_dev, kind):
    q, s = fq.fp8_quant_blockwise(x_dev, KINDS[kind])
    torch.cuda.synchronize()
    return host(q), host(s)


def _check(x_f32, x_dev, kind):
    q, s = _gpu_quant(x_dev, kind)
    qo, so = oracle.quantize(x_f32, kind)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), "scale bits differ"
    bad = np.argwhere(q != qo)
    assert bad.size == 0, "codes differ at %s (gpu %s, oracle %s)" % (
        bad[:5].tolist(), q[tuple(bad[0])], qo[tuple(bad[0])])


def _wide_range_bf16(rows, cols, seed):
    """Per-row exponent window from bf16-subnormal to huge, element offsets
    up to 2^-40 below the row max: exercises every code, underflow, subnormal
    and zero scales."""
    g = np.random.Generator(np.random.PCG64(seed))
    e_row = g.integers(-133, 120, size=(rows, 1))
    e = e_row - g.integers(0, 40, size=(rows, cols))
    mant = g.integers(0, 128, size=(rows, cols))
    sign = g.integers(0, 2, size=(rows, cols))
    e = np.clip(e, -133, 127)
    bits = np.where(e >= -126, ((e + 127) << 7) | mant, (mant | 0x80) >> np.clip(-126 - e, 0, 8))
    bits = (bits | (sign << 15)).astype(np.uint16)
    bits[g.random((rows, cols)) < 0.02] = 0x8000    # some -0
    return bits


@pytest.mark.parametrize("kind", ["row", "block", "tensor"])
def test_all_bf16_patterns(kind):
    g = np.random.Generator(np.random.PCG64(1))
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allb[(allb & 0x7F80) != 0x7F80]
    bits = g.permutation(finite)
    bits = np.concatenate([bits, np.zeros(-bits.size % 512, np.uint16)]).reshape(-1, 512)
    x = synthetic.bf16_to_f32(bits)
    _check(x, to_dev_bf16(bits), kind)


@pytest.mark.parametrize("kind", ["row", "block"])
def test_wide_exponent_range(kind):
    bits = _wide_range_bf16(1024, 640, 2)
    _check(synthetic.bf16_to_f32(bits), to_dev_bf16(bits), kind)


def test_fp32_subnormal_and_zero_tiles():
    x = np.zeros((4, 512), np.float32)
    x[0, :128] = -0.0
    x[1, 128] = 1e-45                      # amax/448 underflows: s = 0
    x[1, 129] = -1e-45
    x[2, 256:384] = np.float32(1e-38) * np.linspace(-1, 1, 128, dtype=np.float32)   # subnormal s
    x[3, 384:] = np.float32(3e-28) * np.linspace(-1, 1, 128, dtype=np.float32)     # s near 2^-90
    x[3, :128] = np.float32(2.0 ** -90 * 448) * np.linspace(-1, 1, 128, dtype=np.float32)
    for kind in ["row", "block", "tensor"]:
        _check(x, to_dev(x), kind)


def test_codes_round_trip():
    g = np.random.Generator(np.random.PCG64(3))
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    codes = g.choice(finite, size=(512, 128))
    codes[np.arange(512), g.integers(0, 128, 512)] = 0x7E
    x = oracle.e4m3_decode(codes)
    q, s = _gpu_quant(to_dev(x), "row")
    assert np.all(s == 1.0)
    assert np.array_equal(q, codes)


@pytest.mark.parametrize("shape", [(1, 1), (3, 300), (129, 130), (300, 200), (257, 1000), (1, 4096)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["row", "block", "tensor"])
def test_ragged_shapes(shape, dtype, kind):
    seed = 10 + shape[0] * 7 + shape[1]
    xf = synthetic.with_outliers_f32(synthetic.normal_f32(shape, seed), 0.01, 100.0, seed + 1)
    if dtype == "bf16":
        bits = synthetic.bf16_from_f32(xf)
        _check(synthetic.bf16_to_f32(bits), to_dev_bf16(bits), kind)
    else:
        _check(xf, to_dev(xf), kind)


@pytest.mark.parametrize("kind", ["row", "block"])
def test_canaries_and_strides(kind):
    rows, cols = 200, 300
    xf = synthetic.normal_f32((rows, cols), 20)
    bits = synthetic.bf16_from_f32(xf)
    xbuf = torch.zeros((rows, 320), dtype=torch.bfloat16, device=DEV)
    xbuf[:, :cols] = to_dev_bf16(bits)
    x = xbuf[:, :cols]                                   # ldx = 320
    qbuf, q = padded(rows, cols, 336, torch.uint8, 0xA5)
    tc = -(-cols // 128)
    srows = rows if kind == "row" else -(-rows // 128)
    sbuf, s = padded(srows, tc, 5, torch.float32, -7.0)
    fq.fp8_quant_blockwise(x, KINDS[kind], q=q, s=s)
    torch.cuda.synchronize()
    assert_canary(qbuf, rows, cols, 0xA5)
    assert_canary(sbuf, srows, tc, -7.0)
    qo, so = oracle.quantize(synthetic.bf16_to_f32(bits), kind)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)


def test_empty_inputs():
    for shape in [(0, 128), (5, 0), (0, 0)]:
        x = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        q, s = fq.fp8_quant_blockwise(x, fq.ROW_1x128)
        torch.cuda.synchronize()
        assert q.shape == shape


def test_tiny_linear_fp32_inputs():
    x, w = synthetic.tiny_linear()
    _check(x, to_dev(x), "row")
    _check(w, to_dev(w), "block")


def test_mlp_forward_full_size():
    x, w = synthetic.mlp_forward()
    _check(synthetic.bf16_to_f32(x), to_dev_bf16(x), "row")
    _check(synthetic.bf16_to_f32(w), to_dev_bf16(w), "block")


def test_long_k_full_size_blockwise_and_tensor():
    x, w = synthetic.long_k()
    xf = synthetic.bf16_to_f32(x)
    xd = to_dev_bf16(x)
    _check(xf, xd, "row")
    _check(xf, xd, "tensor")
    wf = synthetic.bf16_to_f32(w)
    wd = to_dev_bf16(w)
    _check(wf, wd, "block")
    _check(wf, wd, "tensor")


def test_deterministic():
    bits = _wide_range_bf16(512, 1024, 4)
    xd = to_dev_bf16(bits)
    for kind in KINDS:
        a = _gpu_quant(xd, kind)
        b = _gpu_quant(xd, kind)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
