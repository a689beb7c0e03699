"""Helpers for the GPU parity tests: host <-> device copies and comparisons.

Inputs come from ``synthetic`` (seeded numpy), expected values from
``oracle`` (CPU); nothing here computes a quantization or a GEMM.
"""
import numpy as np
import torch

DEV = "cuda:0"


def _aligned_2d(t: torch.Tensor) -> torch.Tensor:
    """Copy a 2-D host tensor to the device with its row stride rounded up to
    16 bytes (the ABI's alignment rule); returns the [rows, cols] view."""
    rows, cols = t.shape
    per = max(1, 16 // t.element_size())
    ld = max(per, -(-cols // per) * per)
    buf = torch.zeros((rows, ld), dtype=t.dtype, device=DEV)
    buf[:, :cols] = t.to(DEV)
    return buf[:, :cols]


def to_dev(a: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return _aligned_2d(t) if t.dim() == 2 else t.to(DEV)


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)
    return _aligned_2d(t) if t.dim() == 2 else t.to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def padded(rows: int, cols: int, ld: int, dtype, fill) -> torch.Tensor:
    """[rows, cols] view of a [rows + 1, ld] buffer pre-filled with a canary."""
    buf = torch.full((rows + 1, ld), fill, dtype=dtype, device=DEV)
    return buf, buf[:rows, :cols]


def assert_canary(buf: torch.Tensor, rows: int, cols: int, fill) -> None:
    b = buf.cpu()
    assert torch.all(b[:rows, cols:] == fill), "write past the last column"
    assert torch.all(b[rows:] == fill), "write past the last row"


def gemm_parity(c_gpu: np.ndarray, c_orc: np.ndarray, R: np.ndarray, tol: float = 1e-3) -> float:
    """|C_gpu - C_oracle| <= tol * R elementwise, R = sum of |products| * |scales|;
    where R == 0 the result must be exactly 0.  Returns max |diff| / R."""
    diff = np.abs(c_gpu.astype(np.float64) - c_orc.astype(np.float64))
    assert np.all(np.isfinite(c_gpu))
    zero = R == 0
    assert np.all(diff[zero] == 0)
    ratio = np.where(zero, 0.0, diff / np.where(zero, 1.0, R))
    worst = float(ratio.max()) if ratio.size else 0.0
    assert worst <= tol, "max |diff|/R = %g" % worst
    return worst


def bf16_parity(c_bf16_bits: np.ndarray, c_gpu_f32: np.ndarray, c_orc: np.ndarray, R: np.ndarray,
                rne_of_gpu_f32: np.ndarray, tol: float = 1e-3) -> None:
    """bf16 output checks: (1) it is exactly the fp32 output of the same GEMM
    rounded to nearest even (``rne_of_gpu_f32``, computed by the oracle's
    rounding routine); (2) its value lies within tol * R plus half a bf16 ulp
    (2^-8 relative) of the oracle's fp32 result."""
    assert np.array_equal(c_bf16_bits, rne_of_gpu_f32), "bf16 output is not RNE of the fp32 result"
    val = (c_bf16_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    co = c_orc.astype(np.float64)
    bound = tol * R + 2.0 ** -8 * (np.abs(co) + tol * R)
    assert np.all(np.abs(val - co) <= bound), "bf16 output outside tolerance"
