"""Block-scaled FP8 (E4M3) quantization and FP8 GEMM on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libfp8q.so`` (declared in
``include/fp8q.h``).  The functions carry the C names and only marshal
arguments: torch supplies device memory and the current stream, every step
of the computation runs in the HIP kernels.  There is no fallback: if the
library is missing the import of this module raises.

Codes are ``torch.uint8`` tensors holding OCP E4M3FN bytes (view them as
``torch.float8_e4m3fn`` if desired); scales are ``torch.float32``, or, for
the ``*_e8m0`` functions, ``torch.uint8`` E8M0 exponent bytes of power-of-two
scales (2^(byte - 127)) whose row stride is a multiple of 4.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8q.so")

# enums of include/fp8q.h
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_DEVICE, ERR_LAUNCH = range(7)
F32, BF16 = 0, 1
ROW_1x128, BLOCK_128x128, TENSOR = 0, 1, 2
B_NK, B_KN = 0, 1

TILE = 128

if not os.path.exists(LIB_PATH):
    raise ImportError(
        "libfp8q.so is not built (expected at %s); run "
        "`python fp8_precision_quant_amd/build.py`" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)
_i64, _int, _p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
_lib.fp8_quant_blockwise.argtypes = [_p, _int, _i64, _i64, _i64, _int, _p, _i64, _p, _i64, _p]
_lib.fp8_quant_transpose.argtypes = [_p, _int, _i64, _i64, _i64,
                                     _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_lib.fp8_gemm_blockscaled.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _int,
                                      _p, _i64, _int, _p, _i64, _int, _p, _i64, _int, _p]
_lib.fp8_grouped_gemm.argtypes = [_i64, _i64, _i64, _i64, _p, _i64, _p, _i64, _p,
                                  _p, _p, _p, _i64, _int, _p]
_lib.fp8_gemm_blockscaled_e4m3.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, _int,
                                           _p, _i64, _int, _p, _i64, _int, _p, _i64, _p, _i64, _p]
_lib.fp8_grouped_gemm_e4m3.argtypes = [_i64, _i64, _i64, _i64, _p, _i64, _p, _i64, _p,
                                       _p, _p, _p, _i64, _p, _i64, _p]
_lib.fp8_grouped_gemm_dgrad.argtypes = [_i64, _i64, _i64, _i64, _p, _i64, _p, _i64, _p,
                                        _p, _p, _p, _i64, _int, _p]
_lib.fp8_grouped_gemm_wgrad.argtypes = [_i64, _i64, _i64, _i64, _p, _i64, _p, _i64,
                                        _p, _i64, _p, _i64, _p, _p, _i64, _p]
_lib.fp8_quant_blockwise_e8m0.argtypes = [_p, _int, _i64, _i64, _i64, _int, _p, _i64, _p, _i64, _p]
_lib.fp8_quant_transpose_e8m0.argtypes = [_p, _int, _i64, _i64, _i64,
                                          _p, _i64, _p, _i64, _p, _i64, _p, _i64, _p]
_lib.fp8_gemm_e8m0.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64,
                               _p, _i64, _int, _p, _i64, _int, _p, _i64, _int, _p]
_d = ctypes.c_double
_lib.fp8_adam_step.argtypes = [_i64, _p, _p, _int, _p, _p, _p, _p, _d, _d, _d, _d, _d, _i64, _p]
for _f in ("fp8_quant_blockwise", "fp8_quant_transpose", "fp8_gemm_blockscaled",
           "fp8_gemm_blockscaled_e4m3", "fp8_grouped_gemm", "fp8_grouped_gemm_e4m3", "fp8_grouped_gemm_dgrad",
           "fp8_grouped_gemm_wgrad", "fp8_quant_blockwise_e8m0", "fp8_quant_transpose_e8m0",
           "fp8_gemm_e8m0", "fp8_adam_step"):
    getattr(_lib, _f).restype = _int
_lib.fp8q_status_string.argtypes = [_int]
_lib.fp8q_status_string.restype = ctypes.c_char_p

SYMBOLS = ("fp8_quant_blockwise", "fp8_quant_transpose", "fp8_gemm_blockscaled",
           "fp8_gemm_blockscaled_e4m3", "fp8_grouped_gemm", "fp8_grouped_gemm_e4m3", "fp8_grouped_gemm_dgrad", "fp8_grouped_gemm_wgrad",
           "fp8_quant_blockwise_e8m0", "fp8_quant_transpose_e8m0", "fp8_gemm_e8m0",
           "fp8_adam_step", "fp8q_status_string")


class Fp8qError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s" % (where, fp8q_status_string(status)))


def fp8q_status_string(status: int) -> str:
    return _lib.fp8q_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise Fp8qError(status, where)


def _stream(device: torch.device, stream) -> int:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(device).cuda_stream


# ---------------------------------------------------------------------------
# argument checks: every tensor handed to the library must be a GPU tensor on
# the device the work is enqueued on, of the dtype the kernel reads, and at
# least as large as the extents the kernel derives from the sizes (the kernels
# trust those extents).  Violations raise ValueError before any launch.
# ---------------------------------------------------------------------------

_CODE_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _device(first: torch.Tensor, stream) -> torch.device:
    """The device the call runs on: the given stream's, else the first operand's."""
    dev = getattr(stream, "device", None)
    dev = torch.device(dev) if dev is not None else first.device
    if dev.type != "cuda":
        raise ValueError("operands must be GPU tensors, got a tensor on %s" % dev)
    return dev


def _on(dev: torch.device, **tensors) -> None:
    for name, t in tensors.items():
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise ValueError("%s must be a torch.Tensor" % name)
        if t.device.type != "cuda" or (dev.index is not None and t.device.index != dev.index):
            raise ValueError("%s is on %s, the call runs on %s" % (name, t.device, dev))


def _dtype(name: str, t: Optional[torch.Tensor], allowed) -> None:
    if t is not None and t.dtype not in allowed:
        raise ValueError("%s must be %s, got %s" % (name, " or ".join(str(a) for a in allowed), t.dtype))


def _min_shape(name: str, t: torch.Tensor, rows: int, cols: int) -> None:
    """A 2-D grid with at least `rows` x `cols` entries (row stride from _ld)."""
    if t.dim() != 2 or t.size(0) < rows or t.size(1) < cols:
        raise ValueError("%s must be at least [%d, %d], got %s" % (name, rows, cols, tuple(t.shape)))


def _shape(name: str, t: torch.Tensor, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _a_scales(name: str, t: torch.Tensor, kind: int, M: int, KB: int) -> int:
    """Scale grid of A (1x128 rows or one per tensor); returns its row stride."""
    if kind == TENSOR:
        if t.numel() < 1:
            raise ValueError("%s: a per-tensor scale needs one element" % name)
        return _ld(t) if t.dim() == 2 else 1
    _min_shape(name, t, M, KB)
    return _ld(t)


def _b_scales(name: str, t: torch.Tensor, kind: int, layout: int, N: int, KB: int) -> int:
    """Scale grid of B for `kind` and `layout`; returns its row stride."""
    NB = _cdiv(N, TILE)
    if kind == TENSOR:
        if t.numel() < 1:
            raise ValueError("%s: a per-tensor scale needs one element" % name)
        return _ld(t) if t.dim() == 2 else 1
    if kind == ROW_1x128:
        _min_shape(name, t, N, KB)
    elif layout == B_NK:
        _min_shape(name, t, NB, KB)
    else:
        _min_shape(name, t, KB, NB)
    return _ld(t)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _ld(t: torch.Tensor) -> int:
    """Row stride (elements) of a 2-D tensor with unit column stride."""
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with contiguous rows, got shape %s strides %s"
                         % (tuple(t.shape), t.stride()))
    return t.stride(0) if t.size(0) > 1 else max(t.stride(0), t.size(1))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError("unsupported input dtype %s" % t.dtype)


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _empty_aligned(rows: int, cols: int, dtype, device, align_elems: int) -> torch.Tensor:
    """[rows, cols] view with a row stride rounded up to `align_elems`."""
    ld = _cdiv(max(cols, 1), align_elems) * align_elems
    return torch.empty((rows, ld), dtype=dtype, device=device)[:, :cols]


def fp8_quant_blockwise(x: torch.Tensor, kind: int = ROW_1x128, q: Optional[torch.Tensor] = None,
                        s: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Quantize ``x[rows, cols]`` (bf16 or fp32) to E4M3 codes and fp32 scales.

    ``kind``: ROW_1x128 -> s[rows, ceil(cols/128)]; BLOCK_128x128 ->
    s[ceil(rows/128), ceil(cols/128)]; TENSOR -> s[1, 1].
    """
    rows, cols = x.shape
    dev = _device(x, stream)
    _on(dev, x=x, q=q, s=s)
    _dtype("x", x, (torch.bfloat16, torch.float32))
    if kind not in (ROW_1x128, BLOCK_128x128, TENSOR):
        raise ValueError("unknown scale kind %r" % (kind,))
    shape = {ROW_1x128: (rows, _cdiv(cols, TILE)),
             BLOCK_128x128: (_cdiv(rows, TILE), _cdiv(cols, TILE)),
             TENSOR: (1, 1)}[kind]
    if q is None:
        q = _empty_aligned(rows, cols, torch.uint8, x.device, 16)
    if s is None:
        s = torch.empty(shape, dtype=torch.float32, device=x.device)
    _dtype("q", q, _CODE_DTYPES)
    _dtype("s", s, (torch.float32,))
    _shape("q", q, (rows, cols))
    if kind == TENSOR:
        if s.numel() < 1:
            raise ValueError("s: a per-tensor scale needs one element")
    else:
        _min_shape("s", s, *shape)
    st = _lib.fp8_quant_blockwise(_ptr(x), _dtype_code(x), rows, cols, _ld(x), kind,
                                  _ptr(q), _ld(q), _ptr(s), _ld(s) if s.dim() == 2 else 1,
                                  _stream(x.device, stream))
    _check(st, "fp8_quant_blockwise")
    return q, s


def _transpose_outputs(dev, x, q_row, s_row, q_colT, s_colT, scale_dtypes, sname="s") -> None:
    R, C = x.shape
    _on(dev, x=x, q_row=q_row, s_row=s_row, q_colT=q_colT, s_colT=s_colT)
    for name, q in (("q_row", q_row), ("q_colT", q_colT)):
        _dtype(name, q, _CODE_DTYPES)
    for name, t in ((sname + "_row", s_row), (sname + "_colT", s_colT)):
        _dtype(name, t, scale_dtypes)
    if (q_row is None) != (s_row is None) or (q_colT is None) != (s_colT is None):
        raise ValueError("each output pair (codes, scales) is given or skipped as a whole")
    if q_row is not None:
        _shape("q_row", q_row, (R, C))
        _min_shape(sname + "_row", s_row, R, _cdiv(C, TILE))
    if q_colT is not None:
        _shape("q_colT", q_colT, (C, R))
        _min_shape(sname + "_colT", s_colT, C, _cdiv(R, TILE))


def fp8_quant_transpose(x: torch.Tensor, rows_out: bool = True, cols_out: bool = True,
                        out: Optional[tuple] = None, stream=None):
    """One read of ``x[R, C]`` -> (q_row[R, C], s_row[R, ceil(C/128)],
    q_colT[C, R], s_colT[C, ceil(R/128)]); a skipped pair is returned as None."""
    R, C = x.shape
    dev = _device(x, stream)
    _dtype("x", x, (torch.bfloat16, torch.float32))
    if out is not None:
        q_row, s_row, q_colT, s_colT = out
    else:
        q_row = _empty_aligned(R, C, torch.uint8, x.device, 16) if rows_out else None
        s_row = torch.empty((R, _cdiv(C, TILE)), dtype=torch.float32, device=x.device) if rows_out else None
        q_colT = _empty_aligned(C, R, torch.uint8, x.device, 16) if cols_out else None
        s_colT = torch.empty((C, _cdiv(R, TILE)), dtype=torch.float32, device=x.device) if cols_out else None
    _transpose_outputs(dev, x, q_row, s_row, q_colT, s_colT, (torch.float32,))
    st = _lib.fp8_quant_transpose(
        _ptr(x), _dtype_code(x), R, C, _ld(x),
        _ptr(q_row), _ld(q_row) if q_row is not None else 0,
        _ptr(s_row), _ld(s_row) if s_row is not None else 0,
        _ptr(q_colT), _ld(q_colT) if q_colT is not None else 0,
        _ptr(s_colT), _ld(s_colT) if s_colT is not None else 0,
        _stream(x.device, stream))
    _check(st, "fp8_quant_transpose")
    return q_row, s_row, q_colT, s_colT


# ---------------------------------------------------------------------------
# power-of-two (E8M0) scales
# ---------------------------------------------------------------------------

def fp8_quant_blockwise_e8m0(x: torch.Tensor, kind: int = ROW_1x128, q: Optional[torch.Tensor] = None,
                             e: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Quantize ``x[rows, cols]`` with power-of-two tile scales: (codes,
    E8M0 bytes ``e``).  ``kind`` ROW_1x128 -> e[rows, ceil(cols/128)];
    BLOCK_128x128 -> e[ceil(rows/128), ceil(cols/128)] (row stride rounded up
    to 4 bytes, as the GEMM reads it)."""
    rows, cols = x.shape
    dev = _device(x, stream)
    _on(dev, x=x, q=q, e=e)
    _dtype("x", x, (torch.bfloat16, torch.float32))
    if kind not in (ROW_1x128, BLOCK_128x128):
        raise ValueError("E8M0 scales come in ROW_1x128 or BLOCK_128x128 tiles")
    r = rows if kind == ROW_1x128 else _cdiv(rows, TILE)
    if q is None:
        q = _empty_aligned(rows, cols, torch.uint8, x.device, 16)
    if e is None:
        e = _empty_aligned(r, _cdiv(cols, TILE), torch.uint8, x.device, 4)
    _dtype("q", q, _CODE_DTYPES)
    _dtype("e", e, (torch.uint8,))
    _shape("q", q, (rows, cols))
    _min_shape("e", e, r, _cdiv(cols, TILE))
    st = _lib.fp8_quant_blockwise_e8m0(_ptr(x), _dtype_code(x), rows, cols, _ld(x), kind,
                                       _ptr(q), _ld(q), _ptr(e), _ld(e), _stream(x.device, stream))
    _check(st, "fp8_quant_blockwise_e8m0")
    return q, e


def fp8_quant_transpose_e8m0(x: torch.Tensor, rows_out: bool = True, cols_out: bool = True,
                             out: Optional[tuple] = None, stream=None):
    """``fp8_quant_transpose`` with power-of-two scales: (q_row, e_row,
    q_colT, e_colT), the ``e`` grids uint8 E8M0 bytes."""
    R, C = x.shape
    dev = _device(x, stream)
    _dtype("x", x, (torch.bfloat16, torch.float32))
    if out is not None:
        q_row, e_row, q_colT, e_colT = out
    else:
        q_row = _empty_aligned(R, C, torch.uint8, x.device, 16) if rows_out else None
        e_row = _empty_aligned(R, _cdiv(C, TILE), torch.uint8, x.device, 4) if rows_out else None
        q_colT = _empty_aligned(C, R, torch.uint8, x.device, 16) if cols_out else None
        e_colT = _empty_aligned(C, _cdiv(R, TILE), torch.uint8, x.device, 4) if cols_out else None
    _transpose_outputs(dev, x, q_row, e_row, q_colT, e_colT, (torch.uint8,), "e")
    st = _lib.fp8_quant_transpose_e8m0(
        _ptr(x), _dtype_code(x), R, C, _ld(x),
        _ptr(q_row), _ld(q_row) if q_row is not None else 0,
        _ptr(e_row), _ld(e_row) if e_row is not None else 0,
        _ptr(q_colT), _ld(q_colT) if q_colT is not None else 0,
        _ptr(e_colT), _ld(e_colT) if e_colT is not None else 0,
        _stream(x.device, stream))
    _check(st, "fp8_quant_transpose_e8m0")
    return q_row, e_row, q_colT, e_colT


def fp8_gemm_e8m0(a: torch.Tensor, ea: torch.Tensor, b: torch.Tensor, eb: torch.Tensor,
                  eb_kind: int = BLOCK_128x128, b_layout: int = B_NK,
                  out_dtype: torch.dtype = torch.bfloat16, c: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """C[M, N] = block-scaled product with power-of-two scales: ``a[M, K]``
    codes with 1x128 E8M0 row scales ``ea``; ``b`` codes (``[N, K]`` for
    B_NK, ``[K, N]`` for B_KN) with E8M0 scales ``eb`` of ``eb_kind``
    (BLOCK_128x128, or ROW_1x128 for B_NK)."""
    M, K = a.shape
    N = b.shape[0] if b_layout == B_NK else b.shape[1]
    if (b.shape[1] if b_layout == B_NK else b.shape[0]) != K:
        raise ValueError("contraction sizes differ: a %s, b %s" % (tuple(a.shape), tuple(b.shape)))
    dev = _device(a, stream)
    _on(dev, a=a, ea=ea, b=b, eb=eb, c=c)
    _dtype("a", a, _CODE_DTYPES)
    _dtype("b", b, _CODE_DTYPES)
    _dtype("ea", ea, (torch.uint8,))
    _dtype("eb", eb, (torch.uint8,))
    if b_layout not in (B_NK, B_KN) or eb_kind not in (ROW_1x128, BLOCK_128x128):
        raise ValueError("unknown layout or scale kind")
    KB = _cdiv(K, TILE)
    if K > 0:
        _min_shape("ea", ea, M, KB)
        ldeb = _b_scales("eb", eb, eb_kind, b_layout, N, KB)
    else:
        ldeb = _ld(eb)
    if c is None:
        c = _empty_aligned(M, N, out_dtype, a.device, 16 // (4 if out_dtype == torch.float32 else 2))
    if c.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("output dtype must be float32 or bfloat16")
    _shape("c", c, (M, N))
    cd = F32 if c.dtype == torch.float32 else BF16
    st = _lib.fp8_gemm_e8m0(M, N, K, _ptr(a), _ld(a), _ptr(ea), _ld(ea),
                            _ptr(b), _ld(b), b_layout, _ptr(eb), ldeb, eb_kind,
                            _ptr(c), _ld(c), cd, _stream(a.device, stream))
    _check(st, "fp8_gemm_e8m0")
    return c


def fp8_adam_state(n: int, device) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """A fresh (all-zero) FP8 moment state for ``n`` parameters:
    (mq[n] uint8, ms[ceil(n/128)] fp32, vq[n], vs[ceil(n/128)])."""
    nb = _cdiv(n, TILE)
    return (torch.zeros(n, dtype=torch.uint8, device=device), torch.zeros(nb, dtype=torch.float32, device=device),
            torch.zeros(n, dtype=torch.uint8, device=device), torch.zeros(nb, dtype=torch.float32, device=device))


def fp8_adam_step(p: torch.Tensor, g: torch.Tensor, state, lr: float, beta1: float = 0.9,
                  beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0, step: int = 1,
                  stream=None) -> None:
    """One AdamW step in place on fp32 parameters ``p`` (any shape,
    contiguous) with gradient ``g`` (same number of elements, fp32 or bf16,
    contiguous) and FP8 moments ``state = (mq, ms, vq, vs)`` (see
    ``fp8_adam_state``)."""
    mq, ms, vq, vs = state
    n = p.numel()
    if g.numel() != n or mq.numel() != n or vq.numel() != n or ms.numel() != _cdiv(n, TILE) \
            or vs.numel() != ms.numel():
        raise ValueError("parameter, gradient and state sizes differ")
    dev = _device(p, stream)
    _on(dev, p=p, g=g, mq=mq, ms=ms, vq=vq, vs=vs)
    for t in (p, g, mq, ms, vq, vs):
        if not t.is_contiguous():
            raise ValueError("fp8_adam_step needs contiguous tensors")
    if p.dtype != torch.float32 or mq.dtype != torch.uint8 or vq.dtype != torch.uint8 \
            or ms.dtype != torch.float32 or vs.dtype != torch.float32:
        raise ValueError("parameters and scales are float32, codes uint8")
    _dtype("g", g, (torch.float32, torch.bfloat16))
    st = _lib.fp8_adam_step(n, _ptr(p), _ptr(g), _dtype_code(g), _ptr(mq), _ptr(ms), _ptr(vq), _ptr(vs),
                            lr, beta1, beta2, eps, weight_decay, step, _stream(p.device, stream))
    _check(st, "fp8_adam_step")


def _gemm_operands(a, sa, sa_kind, b, sb, sb_kind, b_layout, M, N, K, stream):
    """Checks of a dense GEMM's operands; returns the scale grids' row strides."""
    dev = _device(a, stream)
    _on(dev, a=a, sa=sa, b=b, sb=sb)
    _dtype("a", a, _CODE_DTYPES)
    _dtype("b", b, _CODE_DTYPES)
    _dtype("sa", sa, (torch.float32,))
    _dtype("sb", sb, (torch.float32,))
    if sa_kind not in (ROW_1x128, TENSOR) or sb_kind not in (ROW_1x128, BLOCK_128x128, TENSOR) \
            or b_layout not in (B_NK, B_KN):
        raise ValueError("unknown scale kind or layout")
    KB = _cdiv(K, TILE)
    if K == 0:
        return (_ld(sa) if sa.dim() == 2 else 1), (_ld(sb) if sb.dim() == 2 else 1)
    return _a_scales("sa", sa, sa_kind, M, KB), _b_scales("sb", sb, sb_kind, b_layout, N, KB)


def fp8_gemm_blockscaled(a: torch.Tensor, sa: torch.Tensor, sa_kind: int,
                         b: torch.Tensor, sb: torch.Tensor, sb_kind: int, b_layout: int = B_NK,
                         out_dtype: torch.dtype = torch.bfloat16, c: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """C[M, N] = block-scaled product of ``a[M, K]`` codes and ``b`` codes
    (``b[N, K]`` for B_NK, ``b[K, N]`` for B_KN) with their scale grids."""
    M, K = a.shape
    N = b.shape[0] if b_layout == B_NK else b.shape[1]
    if (b.shape[1] if b_layout == B_NK else b.shape[0]) != K:
        raise ValueError("contraction sizes differ: a %s, b %s" % (tuple(a.shape), tuple(b.shape)))
    ldsa, ldsb = _gemm_operands(a, sa, sa_kind, b, sb, sb_kind, b_layout, M, N, K, stream)
    if c is None:
        c = _empty_aligned(M, N, out_dtype, a.device, 16 // (4 if out_dtype == torch.float32 else 2))
    _on(_device(a, stream), c=c)
    if c.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("output dtype must be float32 or bfloat16")
    _shape("c", c, (M, N))
    cd = F32 if c.dtype == torch.float32 else BF16
    st = _lib.fp8_gemm_blockscaled(M, N, K, _ptr(a), _ld(a), _ptr(sa), ldsa, sa_kind,
                                   _ptr(b), _ld(b), b_layout, _ptr(sb), ldsb, sb_kind,
                                   _ptr(c), _ld(c), cd, _stream(a.device, stream))
    _check(st, "fp8_gemm_blockscaled")
    return c


def fp8_gemm_blockscaled_e4m3(a: torch.Tensor, sa: torch.Tensor, sa_kind: int,
                              b: torch.Tensor, sb: torch.Tensor, sb_kind: int, b_layout: int = B_NK,
                              out: Optional[tuple] = None, stream=None):
    """The block-scaled product stored quantized: (codes[M, N] uint8,
    scales[M, ceil(N/128)] float32), the 1x128 quantization of the fp32
    result along N."""
    M, K = a.shape
    N = b.shape[0] if b_layout == B_NK else b.shape[1]
    if (b.shape[1] if b_layout == B_NK else b.shape[0]) != K:
        raise ValueError("contraction sizes differ: a %s, b %s" % (tuple(a.shape), tuple(b.shape)))
    ldsa, ldsb = _gemm_operands(a, sa, sa_kind, b, sb, sb_kind, b_layout, M, N, K, stream)
    if out is not None:
        q, s = out
    else:
        q = _empty_aligned(M, N, torch.uint8, a.device, 16)
        s = torch.empty((M, _cdiv(N, TILE)), dtype=torch.float32, device=a.device)
    _on(_device(a, stream), q=q, s=s)
    _dtype("q", q, _CODE_DTYPES)
    _dtype("s", s, (torch.float32,))
    _shape("q", q, (M, N))
    _min_shape("s", s, M, _cdiv(N, TILE))
    st = _lib.fp8_gemm_blockscaled_e4m3(M, N, K, _ptr(a), _ld(a), _ptr(sa), ldsa, sa_kind,
                                        _ptr(b), _ld(b), b_layout, _ptr(sb), ldsb, sb_kind,
                                        _ptr(q), _ld(q), _ptr(s), _ld(s), _stream(a.device, stream))
    _check(st, "fp8_gemm_blockscaled_e4m3")
    return q, s


def fp8_grouped_gemm(a: torch.Tensor, sa: torch.Tensor, group_offsets: torch.Tensor,
                     b: torch.Tensor, sb: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                     c: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Per group e: rows [off[e], off[e+1]) of ``a[M_pad, K]`` times ``b[e]``
    (``b[G, N, K]`` codes, ``sb[G, ceil(N/128), ceil(K/128)]`` scales);
    ``group_offsets`` is an int32 device tensor of G+1 entries."""
    M_pad, K = a.shape
    G, N, Kb = b.shape
    if Kb != K:
        raise ValueError("contraction sizes differ")
    if group_offsets.dtype != torch.int32 or group_offsets.numel() != G + 1:
        raise ValueError("group_offsets must be int32 with G+1 entries")
    if not (b.is_contiguous() and sb.is_contiguous() and group_offsets.is_contiguous()):
        raise ValueError("b, sb and group_offsets must be contiguous")
    dev = _device(a, stream)
    _on(dev, a=a, sa=sa, group_offsets=group_offsets, b=b, sb=sb, c=c)
    _dtype("a", a, _CODE_DTYPES)
    _dtype("b", b, _CODE_DTYPES)
    _dtype("sa", sa, (torch.float32,))
    _dtype("sb", sb, (torch.float32,))
    _min_shape("sa", sa, M_pad, _cdiv(K, TILE))
    _shape("sb", sb, (G, _cdiv(N, TILE), _cdiv(K, TILE)))
    if c is None:
        c = _empty_aligned(M_pad, N, out_dtype, a.device, 16 // (4 if out_dtype == torch.float32 else 2))
    if c.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("output dtype must be float32 or bfloat16")
    _on(dev, c=c)
    _shape("c", c, (M_pad, N))
    cd = F32 if c.dtype == torch.float32 else BF16
    st = _lib.fp8_grouped_gemm(G, M_pad, N, K, _ptr(a), _ld(a), _ptr(sa), _ld(sa),
                               _ptr(group_offsets), _ptr(b), _ptr(sb), _ptr(c), _ld(c), cd,
                               _stream(a.device, stream))
    _check(st, "fp8_grouped_gemm")
    return c


def fp8_grouped_gemm_e4m3(a: torch.Tensor, sa: torch.Tensor, group_offsets: torch.Tensor,
                          b: torch.Tensor, sb: torch.Tensor, q: Optional[torch.Tensor] = None,
                          s: Optional[torch.Tensor] = None, stream=None):
    """``fp8_grouped_gemm`` stored quantized: returns ``(q, s)``, the E4M3
    codes ``q[M_pad, N]`` and 1x128 scales ``s[M_pad, ceil(N/128)]`` of the
    result (rows at or past off[G] are not written)."""
    M_pad, K = a.shape
    G, N, Kb = b.shape
    if Kb != K:
        raise ValueError("contraction sizes differ")
    if group_offsets.dtype != torch.int32 or group_offsets.numel() != G + 1:
        raise ValueError("group_offsets must be int32 with G+1 entries")
    if not (b.is_contiguous() and sb.is_contiguous() and group_offsets.is_contiguous()):
        raise ValueError("b, sb and group_offsets must be contiguous")
    dev = _device(a, stream)
    _on(dev, a=a, sa=sa, group_offsets=group_offsets, b=b, sb=sb, q=q, s=s)
    _dtype("a", a, _CODE_DTYPES)
    _dtype("b", b, _CODE_DTYPES)
    _dtype("sa", sa, (torch.float32,))
    _dtype("sb", sb, (torch.float32,))
    _min_shape("sa", sa, M_pad, _cdiv(K, TILE))
    _shape("sb", sb, (G, _cdiv(N, TILE), _cdiv(K, TILE)))
    if q is None:
        q = _empty_aligned(M_pad, N, torch.uint8, a.device, 16)
    if s is None:
        s = torch.empty((M_pad, _cdiv(N, TILE)), dtype=torch.float32, device=a.device)
    _dtype("q", q, _CODE_DTYPES)
    _dtype("s", s, (torch.float32,))
    _min_shape("q", q, M_pad, N)
    _min_shape("s", s, M_pad, _cdiv(N, TILE))
    st = _lib.fp8_grouped_gemm_e4m3(G, M_pad, N, K, _ptr(a), _ld(a), _ptr(sa), _ld(sa),
                                    _ptr(group_offsets), _ptr(b), _ptr(sb), _ptr(q), _ld(q), _ptr(s),
                                    _ld(s), _stream(a.device, stream))
    _check(st, "fp8_grouped_gemm_e4m3")
    return q, s


def fp8_grouped_gemm_dgrad(a: torch.Tensor, sa: torch.Tensor, group_offsets: torch.Tensor,
                           w: torch.Tensor, sw: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                           c: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Per group e: rows [off[e], off[e+1]) of ``a[M_pad, N]`` (dY codes,
    1x128 scales along N) times expert weight ``w[e]`` read as stored
    (``w[G, N, K]`` codes, ``sw[G, ceil(N/128), ceil(K/128)]`` block scales):
    dX[M_pad, K]."""
    M_pad, N = a.shape
    G, Nw, K = w.shape
    if Nw != N:
        raise ValueError("contraction sizes differ")
    if group_offsets.dtype != torch.int32 or group_offsets.numel() != G + 1:
        raise ValueError("group_offsets must be int32 with G+1 entries")
    if not (w.is_contiguous() and sw.is_contiguous() and group_offsets.is_contiguous()):
        raise ValueError("w, sw and group_offsets must be contiguous")
    dev = _device(a, stream)
    _on(dev, a=a, sa=sa, group_offsets=group_offsets, w=w, sw=sw, c=c)
    _dtype("a", a, _CODE_DTYPES)
    _dtype("w", w, _CODE_DTYPES)
    _dtype("sa", sa, (torch.float32,))
    _dtype("sw", sw, (torch.float32,))
    _min_shape("sa", sa, M_pad, _cdiv(N, TILE))
    _shape("sw", sw, (G, _cdiv(N, TILE), _cdiv(K, TILE)))
    if c is None:
        c = _empty_aligned(M_pad, K, out_dtype, a.device, 16 // (4 if out_dtype == torch.float32 else 2))
    if c.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("output dtype must be float32 or bfloat16")
    _on(dev, c=c)
    _shape("c", c, (M_pad, K))
    cd = F32 if c.dtype == torch.float32 else BF16
    st = _lib.fp8_grouped_gemm_dgrad(G, M_pad, N, K, _ptr(a), _ld(a), _ptr(sa), _ld(sa),
                                     _ptr(group_offsets), _ptr(w), _ptr(sw), _ptr(c), _ld(c), cd,
                                     _stream(a.device, stream))
    _check(st, "fp8_grouped_gemm_dgrad")
    return c


def fp8_grouped_gemm_wgrad(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor,
                           group_offsets: torch.Tensor, c: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """Per group e: dW[e] = sum over the group's tokens of ``a[N, M_pad]``
    (dY^T codes) times ``b[K, M_pad]`` (X^T codes), both with 1x128 scales
    along tokens (fp8_quant_transpose's column outputs): fp32 dW[G, N, K]."""
    N, M_pad = a.shape
    K, Mb = b.shape
    if Mb != M_pad:
        raise ValueError("token counts differ")
    G = group_offsets.numel() - 1
    if group_offsets.dtype != torch.int32 or G < 1 or not group_offsets.is_contiguous():
        raise ValueError("group_offsets must be a contiguous int32 tensor with G+1 entries")
    dev = _device(a, stream)
    _on(dev, a=a, sa=sa, b=b, sb=sb, group_offsets=group_offsets, c=c)
    _dtype("a", a, _CODE_DTYPES)
    _dtype("b", b, _CODE_DTYPES)
    _dtype("sa", sa, (torch.float32,))
    _dtype("sb", sb, (torch.float32,))
    _min_shape("sa", sa, N, M_pad // TILE)
    _min_shape("sb", sb, K, M_pad // TILE)
    if c is None:
        c = torch.empty((G, N, K), dtype=torch.float32, device=a.device)
    _on(dev, c=c)
    if c.dtype != torch.float32 or c.dim() != 3 or c.shape != (G, N, K) or c.stride(0) != N * c.stride(1) \
            or c.stride(2) != 1:
        raise ValueError("c must be float32 [G, N, K] with group stride N * row stride")
    st = _lib.fp8_grouped_gemm_wgrad(G, M_pad, N, K, _ptr(a), _ld(a), _ptr(sa), _ld(sa),
                                     _ptr(b), _ld(b), _ptr(sb), _ld(sb), _ptr(group_offsets),
                                     _ptr(c), c.stride(1), _stream(a.device, stream))
    _check(st, "fp8_grouped_gemm_wgrad")
    return c
