"""The Python binding's argument checks, on the host (no GPU, no launch).

Every wrapper must reject, with ValueError and before calling the library:
tensors that are not on the GPU the call runs on, codes that are not bytes,
scales of the wrong dtype, and scale grids or outputs smaller than the
extents the kernels derive from the sizes.  The device check is tested with
CPU tensors; the dtype and size checks with the device check bypassed and the
C library replaced by a stub that fails the test if it is reached.
"""
import pytest
import torch

import fp8_precision_quant_amd as fq

u8, f32, bf16 = torch.uint8, torch.float32, torch.bfloat16


def cpu(shape, dtype=f32):
    return torch.zeros(shape, dtype=dtype)


def test_cpu_tensors_are_rejected():
    x = cpu((4, 256), bf16)
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8_quant_blockwise(x)
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8_quant_transpose(x)
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8_quant_blockwise_e8m0(x)
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8_quant_transpose_e8m0(x)
    a, b = cpu((4, 256), u8), cpu((128, 256), u8)
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8_gemm_blockscaled(a, cpu((4, 2)), fq.ROW_1x128, b, cpu((1, 2)), fq.BLOCK_128x128)
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8_gemm_blockscaled_e4m3(a, cpu((4, 2)), fq.ROW_1x128, b, cpu((1, 2)), fq.BLOCK_128x128)
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8_gemm_e8m0(a, cpu((4, 2), u8), b, cpu((1, 2), u8))
    off = torch.tensor([0, 128], dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8_grouped_gemm(cpu((128, 256), u8), cpu((128, 2)), off, cpu((1, 128, 256), u8), cpu((1, 1, 2)))
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8_grouped_gemm_dgrad(cpu((128, 256), u8), cpu((128, 2)), off, cpu((1, 256, 128), u8),
                                  cpu((1, 2, 1)))
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8_grouped_gemm_wgrad(cpu((128, 128), u8), cpu((128, 1)), cpu((128, 128), u8), cpu((128, 1)), off)
    with pytest.raises(ValueError, match="GPU"):
        fq.fp8_adam_step(cpu(256), cpu(256), (cpu(256, u8), cpu(2), cpu(256, u8), cpu(2)), lr=1e-3)


class _NoLib:
    """Stands in for the C library: any call fails the test."""

    def __getattr__(self, name):
        raise AssertionError("the library was called (%s) although the arguments are invalid" % name)


@pytest.fixture
def no_device_check(monkeypatch):
    monkeypatch.setattr(fq, "_device", lambda first, stream: torch.device("cuda", 0))
    monkeypatch.setattr(fq, "_on", lambda dev, **t: None)
    monkeypatch.setattr(fq, "_lib", _NoLib())


def test_dtype_checks(no_device_check):
    M, N, K = 4, 128, 256
    a, b = cpu((M, K), u8), cpu((N, K), u8)
    sa, sb = cpu((M, 2)), cpu((1, 2))
    with pytest.raises(ValueError, match="x must be"):
        fq.fp8_quant_blockwise(cpu((4, 256), torch.float16))
    with pytest.raises(ValueError, match="s must be"):
        fq.fp8_quant_blockwise(cpu((4, 256), bf16), q=cpu((4, 256), u8), s=cpu((4, 2), bf16))
    with pytest.raises(ValueError, match="q must be"):
        fq.fp8_quant_blockwise(cpu((4, 256), bf16), q=cpu((4, 256), torch.int32), s=cpu((4, 2)))
    with pytest.raises(ValueError, match="a must be"):
        fq.fp8_gemm_blockscaled(cpu((M, K), torch.int8), sa, fq.ROW_1x128, b, sb, fq.BLOCK_128x128)
    with pytest.raises(ValueError, match="sa must be"):
        fq.fp8_gemm_blockscaled(a, cpu((M, 2), torch.float16), fq.ROW_1x128, b, sb, fq.BLOCK_128x128)
    with pytest.raises(ValueError, match="sb must be"):
        fq.fp8_gemm_blockscaled(a, sa, fq.ROW_1x128, b, cpu((1, 2), u8), fq.BLOCK_128x128)
    with pytest.raises(ValueError, match="ea must be"):
        fq.fp8_gemm_e8m0(a, sa, b, cpu((1, 2), u8))
    with pytest.raises(ValueError, match="s_colT must be"):
        fq.fp8_quant_transpose(cpu((128, 128), bf16), out=(cpu((128, 128), u8), cpu((128, 1)),
                                                           cpu((128, 128), u8), cpu((128, 1), u8)))
    with pytest.raises(ValueError, match="e_row must be"):
        fq.fp8_quant_transpose_e8m0(cpu((128, 128), bf16), out=(cpu((128, 128), u8), cpu((128, 1)),
                                                                cpu((128, 128), u8), cpu((128, 1), u8)))
    # float8_e4m3fn codes are accepted as bytes (the checks pass, the stub is reached)
    with pytest.raises(AssertionError, match="library was called"):
        fq.fp8_gemm_blockscaled(a.view(torch.float8_e4m3fn), sa, fq.ROW_1x128, b, sb, fq.BLOCK_128x128,
                                c=cpu((M, N)))


def test_extent_checks(no_device_check):
    M, N, K = 300, 384, 512          # KB = 4, NB = 3
    a, b, bkn = cpu((M, K), u8), cpu((N, K), u8), cpu((K, N), u8)
    # A row scales with too few rows / chunks
    with pytest.raises(ValueError, match="sa must be at least"):
        fq.fp8_gemm_blockscaled(a, cpu((1, 4)), fq.ROW_1x128, b, cpu((3, 4)), fq.BLOCK_128x128)
    with pytest.raises(ValueError, match="sa must be at least"):
        fq.fp8_gemm_blockscaled(a, cpu((M, 3)), fq.ROW_1x128, b, cpu((3, 4)), fq.BLOCK_128x128)
    # B block scales: [NB][KB] for NK, [KB][NB] for KN; row scales [N][KB]
    with pytest.raises(ValueError, match="sb must be at least"):
        fq.fp8_gemm_blockscaled(a, cpu((M, 4)), fq.ROW_1x128, b, cpu((2, 4)), fq.BLOCK_128x128)
    with pytest.raises(ValueError, match="sb must be at least"):
        fq.fp8_gemm_blockscaled(a, cpu((M, 4)), fq.ROW_1x128, bkn, cpu((3, 4)), fq.BLOCK_128x128, fq.B_KN)
    with pytest.raises(ValueError, match="sb must be at least"):
        fq.fp8_gemm_blockscaled(a, cpu((M, 4)), fq.ROW_1x128, b, cpu((N - 1, 4)), fq.ROW_1x128)
    with pytest.raises(ValueError, match="sa: a per-tensor"):
        fq.fp8_gemm_blockscaled(a, cpu((0,)), fq.TENSOR, b, cpu((3, 4)), fq.BLOCK_128x128)
    # outputs of the wrong shape
    with pytest.raises(ValueError, match="c must have shape"):
        fq.fp8_gemm_blockscaled(a, cpu((M, 4)), fq.ROW_1x128, b, cpu((3, 4)), fq.BLOCK_128x128,
                                c=cpu((M, N - 1)))
    with pytest.raises(ValueError, match="s must be at least"):
        fq.fp8_gemm_blockscaled_e4m3(a, cpu((M, 4)), fq.ROW_1x128, b, cpu((3, 4)), fq.BLOCK_128x128,
                                     out=(cpu((M, N), u8), cpu((M, 2))))
    with pytest.raises(ValueError, match="s must be at least"):
        fq.fp8_quant_blockwise(cpu((300, 300), bf16), fq.BLOCK_128x128, q=cpu((300, 300), u8), s=cpu((2, 3)))
    with pytest.raises(ValueError, match="q must have shape"):
        fq.fp8_quant_blockwise(cpu((300, 300), bf16), q=cpu((300, 299), u8), s=cpu((300, 3)))
    with pytest.raises(ValueError, match="s_colT must be at least"):
        fq.fp8_quant_transpose(cpu((300, 200), bf16), out=(None, None, cpu((200, 300), u8), cpu((200, 2))))
    with pytest.raises(ValueError, match="given or skipped"):
        fq.fp8_quant_transpose(cpu((300, 200), bf16), out=(cpu((300, 200), u8), None, None, None))
    with pytest.raises(ValueError, match="eb must be at least"):
        fq.fp8_gemm_e8m0(a, cpu((M, 4), u8), b, cpu((3, 3), u8))
    # grouped: expert scale stacks must match [G][NB][KB]
    off = torch.tensor([0, 128, 256], dtype=torch.int32)
    with pytest.raises(ValueError, match="sb must have shape"):
        fq.fp8_grouped_gemm(cpu((256, K), u8), cpu((256, 4)), off, cpu((2, N, K), u8), cpu((2, 3, 3)))
    with pytest.raises(ValueError, match="sa must be at least"):
        fq.fp8_grouped_gemm(cpu((256, K), u8), cpu((128, 4)), off, cpu((2, N, K), u8), cpu((2, 3, 4)))
    with pytest.raises(ValueError, match="sw must have shape"):
        fq.fp8_grouped_gemm_dgrad(cpu((256, N), u8), cpu((256, 3)), off, cpu((2, N, K), u8), cpu((2, 4, 3)))
    with pytest.raises(ValueError, match="sb must be at least"):
        fq.fp8_grouped_gemm_wgrad(cpu((N, 256), u8), cpu((N, 2)), cpu((K, 256), u8), cpu((K - 1, 2)), off)
