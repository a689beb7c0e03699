"""The C-ABI library on the host: it loads, exports every function that
include/fp8q.h declares, and rejects bad arguments with the documented
status before touching a device (no kernel is launched by these tests)."""
import ctypes
import os
import re

import pytest
import torch

import fp8_precision_quant_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert names == sorted(["fp8_quant_blockwise", "fp8_quant_transpose", "fp8_gemm_blockscaled",
                            "fp8_gemm_blockscaled_e4m3", "fp8_grouped_gemm", "fp8_grouped_gemm_e4m3",
                            "fp8_grouped_gemm_dgrad", "fp8_grouped_gemm_wgrad",
                            "fp8_quant_blockwise_e8m0", "fp8_quant_transpose_e8m0", "fp8_gemm_e8m0",
                            "fp8_adam_step", "fp8q_status_string"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fq.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(fq.SYMBOLS) == set(declared_functions())


def test_status_strings():
    for st in range(7):
        assert fq.fp8q_status_string(st).startswith("FP8Q_")
    assert "unknown" in fq.fp8q_status_string(99)


L = fq._lib
A16 = 0x10000          # fake, 16-byte aligned device addresses: never dereferenced
MIS = 0x10004          # misaligned


def q_blockwise(**kw):
    args = dict(x=A16, dt=fq.BF16, rows=4, cols=256, ldx=256, kind=fq.ROW_1x128,
                q=A16, ldq=256, s=A16, lds=2, stream=None)
    args.update(kw)
    return L.fp8_quant_blockwise(args["x"], args["dt"], args["rows"], args["cols"], args["ldx"],
                                 args["kind"], args["q"], args["ldq"], args["s"], args["lds"],
                                 args["stream"])


def test_quant_blockwise_validation():
    assert q_blockwise(dt=7) == fq.ERR_UNSUPPORTED
    assert q_blockwise(kind=9) == fq.ERR_UNSUPPORTED
    assert q_blockwise(rows=-1) == fq.ERR_SHAPE
    assert q_blockwise(rows=0, x=None, q=None, s=None) == fq.OK      # empty: nothing launched
    assert q_blockwise(cols=0, x=None, q=None, s=None) == fq.OK
    assert q_blockwise(x=None) == fq.ERR_NULL
    assert q_blockwise(s=None) == fq.ERR_NULL
    assert q_blockwise(ldx=200) == fq.ERR_SHAPE
    assert q_blockwise(lds=1) == fq.ERR_SHAPE
    assert q_blockwise(kind=fq.BLOCK_128x128, lds=1) == fq.ERR_SHAPE
    assert q_blockwise(x=MIS) == fq.ERR_ALIGN
    assert q_blockwise(q=A16 + 8) == fq.ERR_ALIGN
    assert q_blockwise(ldx=260, cols=256) == fq.ERR_ALIGN             # 520 bytes per row
    assert q_blockwise(ldq=264) == fq.ERR_ALIGN
    # 128x128 blocks are indexed with 31-bit block ids: ceil(rows/128) * ceil(cols/128) < 2^31
    assert q_blockwise(kind=fq.BLOCK_128x128, rows=128 * (1 << 30)) == fq.ERR_SHAPE


def test_quant_transpose_validation():
    f = L.fp8_quant_transpose
    base = [A16, fq.BF16, 256, 384, 384, A16, 384, A16, 3, A16, 256, A16, 2, None]
    def call(**ch):
        a = list(base)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a1=5) == fq.ERR_UNSUPPORTED
    assert call(a2=-3) == fq.ERR_SHAPE
    assert call(a2=0, a0=None) == fq.OK
    assert call(a0=None) == fq.ERR_NULL
    assert call(a5=None) == fq.ERR_NULL                   # half a pair
    assert call(a5=None, a7=None, a9=None, a11=None) == fq.OK   # nothing requested
    assert call(a6=200) == fq.ERR_SHAPE
    assert call(a12=1) == fq.ERR_SHAPE
    assert call(a9=MIS) == fq.ERR_ALIGN
    assert call(a10=264) == fq.ERR_ALIGN


def test_gemm_validation():
    f = L.fp8_gemm_blockscaled
    # M, N, K, a, lda, sa, ldsa, sa_kind, b, ldb, layout, sb, ldsb, sb_kind, c, ldc, cdt, stream
    base = [256, 256, 512, A16, 512, A16, 4, fq.ROW_1x128, A16, 512, fq.B_NK, A16, 4,
            fq.BLOCK_128x128, A16, 256, fq.BF16, None]
    def call(**ch):
        a = list(base)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a16=3) == fq.ERR_UNSUPPORTED
    assert call(a10=2) == fq.ERR_UNSUPPORTED
    assert call(a7=fq.BLOCK_128x128) == fq.ERR_UNSUPPORTED
    assert call(a13=fq.ROW_1x128, a10=fq.B_KN, a9=256) == fq.ERR_UNSUPPORTED
    assert call(a0=-1) == fq.ERR_SHAPE
    assert call(a0=0, a3=None) == fq.OK
    assert call(a3=None) == fq.ERR_NULL
    assert call(a11=None) == fq.ERR_NULL
    assert call(a4=500) == fq.ERR_SHAPE
    assert call(a6=3) == fq.ERR_SHAPE
    assert call(a12=3) == fq.ERR_SHAPE
    assert call(a10=fq.B_KN, a9=128) == fq.ERR_SHAPE      # ldb < N for KN
    assert call(a10=fq.B_KN, a9=256, a12=1) == fq.ERR_SHAPE  # KN grid row stride < ceil(N/128)
    assert call(a15=200) == fq.ERR_SHAPE
    assert call(a3=MIS) == fq.ERR_ALIGN
    assert call(a14=A16 + 4) == fq.ERR_ALIGN
    assert call(a4=520, a2=512) == fq.ERR_ALIGN


def test_grouped_validation():
    f = L.fp8_grouped_gemm
    # G, M_pad, N, K, a, lda, sa, ldsa, off, b, sb, c, ldc, cdt, stream
    base = [4, 512, 256, 256, A16, 256, A16, 2, A16, A16, A16, A16, 256, fq.BF16, None]
    def call(**ch):
        a = list(base)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a13=4) == fq.ERR_UNSUPPORTED
    assert call(a0=0) == fq.ERR_SHAPE
    assert call(a1=500) == fq.ERR_SHAPE                    # M_pad not a multiple of 128
    assert call(a1=0, a4=None) == fq.OK
    assert call(a8=None) == fq.ERR_NULL
    assert call(a7=1) == fq.ERR_SHAPE
    assert call(a3=200, a5=256, a7=2) == fq.ERR_ALIGN      # K % 16 != 0
    assert call(a8=A16 + 2) == fq.ERR_ALIGN
    assert call(a0=1025, a1=1025 * 128) == fq.ERR_UNSUPPORTED   # the offsets live in LDS: G <= 1024


def test_gemm_e4m3_validation():
    f = L.fp8_gemm_blockscaled_e4m3
    # M, N, K, a, lda, sa, ldsa, sa_kind, b, ldb, layout, sb, ldsb, sb_kind, q, ldq, s, lds, stream
    base = [256, 256, 512, A16, 512, A16, 4, fq.ROW_1x128, A16, 512, fq.B_NK, A16, 4,
            fq.BLOCK_128x128, A16, 256, A16, 2, None]
    def call(**ch):
        a = list(base)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a10=2) == fq.ERR_UNSUPPORTED
    assert call(a13=fq.ROW_1x128, a10=fq.B_KN, a9=256) == fq.ERR_UNSUPPORTED
    assert call(a13=fq.ROW_1x128) == fq.ERR_UNSUPPORTED    # row-scaled B: not stored as E4M3
    assert call(a1=0, a14=None) == fq.OK                   # empty output
    assert call(a14=None) == fq.ERR_NULL
    assert call(a16=None) == fq.ERR_NULL
    assert call(a3=None) == fq.ERR_NULL
    assert call(a15=200) == fq.ERR_SHAPE                   # ldq < N
    assert call(a17=1) == fq.ERR_SHAPE                     # lds < ceil(N/128)
    assert call(a6=3) == fq.ERR_SHAPE
    assert call(a15=264) == fq.ERR_ALIGN                   # ldq % 16 != 0
    assert call(a14=A16 + 1) == fq.ERR_ALIGN
    assert call(a3=MIS) == fq.ERR_ALIGN


def test_grouped_e4m3_validation():
    f = L.fp8_grouped_gemm_e4m3
    # G, M_pad, N, K, a, lda, sa, ldsa, off, b, sb, q, ldq, s, lds, stream
    base = [4, 512, 256, 256, A16, 256, A16, 2, A16, A16, A16, A16, 256, A16, 2, None]
    def call(**ch):
        a = list(base)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=0) == fq.ERR_SHAPE
    assert call(a1=500) == fq.ERR_SHAPE                    # M_pad not a multiple of 128
    assert call(a1=0, a4=None) == fq.OK                    # empty output
    assert call(a2=0, a11=None) == fq.OK
    assert call(a3=0) == fq.ERR_UNSUPPORTED                # K must be a positive multiple of 128
    assert call(a3=200, a5=256) == fq.ERR_UNSUPPORTED
    assert call(a8=None) == fq.ERR_NULL
    assert call(a11=None) == fq.ERR_NULL
    assert call(a13=None) == fq.ERR_NULL
    assert call(a5=200) == fq.ERR_SHAPE                    # lda < K
    assert call(a7=1) == fq.ERR_SHAPE                      # ldsa < K/128
    assert call(a12=200) == fq.ERR_SHAPE                   # ldq < N
    assert call(a14=1) == fq.ERR_SHAPE                     # lds < ceil(N/128)
    assert call(a12=264) == fq.ERR_ALIGN                   # ldq % 16 != 0
    assert call(a11=A16 + 1) == fq.ERR_ALIGN
    assert call(a8=A16 + 2) == fq.ERR_ALIGN
    assert call(a0=1025, a1=1025 * 128) == fq.ERR_UNSUPPORTED


def test_grouped_dgrad_validation():
    f = L.fp8_grouped_gemm_dgrad
    # G, M_pad, N, K, a, lda, sa, ldsa, off, w, sw, c, ldc, cdt, stream
    base = [4, 512, 256, 256, A16, 256, A16, 2, A16, A16, A16, A16, 256, fq.BF16, None]
    def call(**ch):
        a = list(base)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a13=4) == fq.ERR_UNSUPPORTED
    assert call(a0=0) == fq.ERR_SHAPE
    assert call(a1=500) == fq.ERR_SHAPE                    # M_pad not a multiple of 128
    assert call(a1=0, a4=None) == fq.OK                    # empty output
    assert call(a3=0, a11=None) == fq.OK
    assert call(a8=None) == fq.ERR_NULL
    assert call(a9=None) == fq.ERR_NULL
    assert call(a5=200) == fq.ERR_SHAPE                    # lda < N
    assert call(a7=1) == fq.ERR_SHAPE                      # ldsa < ceil(N/128)
    assert call(a12=200) == fq.ERR_SHAPE                   # ldc < K
    assert call(a3=200, a12=256) == fq.ERR_ALIGN           # K % 16 != 0 (weight row stride)
    assert call(a8=A16 + 2) == fq.ERR_ALIGN
    assert call(a0=1025, a1=1025 * 128) == fq.ERR_UNSUPPORTED


def test_grouped_wgrad_validation():
    f = L.fp8_grouped_gemm_wgrad
    # G, M_pad, N, K, a, lda, sa, ldsa, b, ldb, sb, ldsb, off, c, ldc, stream
    base = [4, 512, 256, 256, A16, 512, A16, 4, A16, 512, A16, 4, A16, A16, 256, None]
    def call(**ch):
        a = list(base)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=0) == fq.ERR_SHAPE
    assert call(a1=500) == fq.ERR_SHAPE                    # M_pad not a multiple of 128
    assert call(a2=0, a13=None) == fq.OK                   # empty output
    assert call(a12=None) == fq.ERR_NULL
    assert call(a8=None) == fq.ERR_NULL
    assert call(a5=400) == fq.ERR_SHAPE                    # lda < M_pad
    assert call(a11=3) == fq.ERR_SHAPE                     # ldsb < M_pad/128
    assert call(a14=200) == fq.ERR_SHAPE                   # ldc < K
    assert call(a9=520) == fq.ERR_ALIGN                    # ldb % 16 != 0
    assert call(a13=A16 + 4) == fq.ERR_ALIGN
    assert call(a0=1025, a1=1025 * 128, a5=1025 * 128, a9=1025 * 128, a7=1025, a11=1025) == fq.ERR_UNSUPPORTED


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is present: valid fake pointers would launch")
def test_valid_arguments_without_gpu_report_device_error():
    assert q_blockwise() == fq.ERR_DEVICE


def test_quant_e8m0_validation():
    f = L.fp8_quant_blockwise_e8m0
    # x, dtype, rows, cols, ldx, kind, q, ldq, e, lde, stream
    base = [A16, fq.BF16, 4, 256, 256, fq.ROW_1x128, A16, 256, A16, 2, None]
    def call(**ch):
        a = list(base)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a5=fq.TENSOR) == fq.ERR_UNSUPPORTED         # power-of-two scales are per tile
    assert call(a1=5) == fq.ERR_UNSUPPORTED
    assert call(a2=-1) == fq.ERR_SHAPE
    assert call(a2=0, a0=None) == fq.OK                      # empty input
    assert call(a8=None) == fq.ERR_NULL
    assert call(a9=1) == fq.ERR_SHAPE                        # lde < ceil(cols/128)
    assert call(a7=200) == fq.ERR_SHAPE
    assert call(a0=MIS) == fq.ERR_ALIGN
    assert call(a7=264) == fq.ERR_ALIGN
    g = L.fp8_quant_transpose_e8m0
    # x, dtype, rows, cols, ldx, q_row, ldq_row, e_row, lde_row, q_colT, ldq_colT, e_colT, lde_colT, stream
    tb = [A16, fq.BF16, 256, 256, 256, A16, 256, A16, 2, A16, 256, A16, 2, None]
    def tcall(**ch):
        a = list(tb)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return g(*a)
    assert tcall(a7=None) == fq.ERR_NULL                     # half of the row pair
    assert tcall(a5=None, a7=None, a9=None, a11=None) == fq.OK
    assert tcall(a12=1) == fq.ERR_SHAPE
    assert tcall(a10=200) == fq.ERR_SHAPE
    assert tcall(a9=MIS) == fq.ERR_ALIGN


def test_gemm_e8m0_validation():
    f = L.fp8_gemm_e8m0
    # M, N, K, a, lda, ea, ldea, b, ldb, layout, eb, ldeb, eb_kind, c, ldc, cdt, stream
    base = [256, 256, 512, A16, 512, A16, 4, A16, 512, fq.B_NK, A16, 4, fq.BLOCK_128x128,
            A16, 256, fq.BF16, None]
    def call(**ch):
        a = list(base)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a15=3) == fq.ERR_UNSUPPORTED
    assert call(a9=2) == fq.ERR_UNSUPPORTED
    assert call(a12=fq.TENSOR) == fq.ERR_UNSUPPORTED
    assert call(a12=fq.ROW_1x128, a9=fq.B_KN, a8=256) == fq.ERR_UNSUPPORTED
    assert call(a0=0, a13=None) == fq.OK                     # empty output
    assert call(a13=None) == fq.ERR_NULL
    assert call(a5=None) == fq.ERR_NULL
    assert call(a10=None) == fq.ERR_NULL
    assert call(a6=3) == fq.ERR_SHAPE                        # ldea < ceil(K/128)
    assert call(a9=fq.B_KN, a8=256, a11=1) == fq.ERR_SHAPE   # KN block grid: ldeb < ceil(N/128)
    assert call(a14=200) == fq.ERR_SHAPE
    assert call(a6=6) == fq.ERR_ALIGN                        # scale rows read as 4-byte words
    assert call(a11=6) == fq.ERR_ALIGN
    assert call(a5=A16 + 2) == fq.ERR_ALIGN
    assert call(a10=A16 + 1) == fq.ERR_ALIGN
    assert call(a3=MIS) == fq.ERR_ALIGN
    assert call(a13=A16 + 4) == fq.ERR_ALIGN


def test_adam_validation():
    f = L.fp8_adam_step
    # n, p, g, g_dtype, mq, ms, vq, vs, lr, beta1, beta2, eps, wd, step, stream
    base = [1000, A16, A16, fq.BF16, A16, A16, A16, A16, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None]
    def call(**ch):
        a = list(base)
        for i, v in ch.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a3=7) == fq.ERR_UNSUPPORTED
    assert call(a9=1.0) == fq.ERR_UNSUPPORTED               # beta1 outside [0, 1)
    assert call(a10=-0.1) == fq.ERR_UNSUPPORTED
    assert call(a13=0) == fq.ERR_UNSUPPORTED                # step < 1: no bias correction
    assert call(a8=float("nan")) == fq.ERR_UNSUPPORTED
    assert call(a11=float("inf")) == fq.ERR_UNSUPPORTED
    assert call(a0=-1) == fq.ERR_SHAPE
    assert call(a0=0, a1=None) == fq.OK                      # nothing to update
    assert call(a1=None) == fq.ERR_NULL
    assert call(a7=None) == fq.ERR_NULL
    assert call(a2=MIS) == fq.ERR_ALIGN
    assert call(a4=A16 + 8) == fq.ERR_ALIGN
    assert call(a5=A16 + 2) == fq.ERR_ALIGN
