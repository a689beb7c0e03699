"""Dense GEMMs with an operand of 2 GiB or more.

The kernel addresses its operands with 32-bit buffer offsets, so the library
cuts such a call into launches over slices of M (rows of A and of C) or, for
a [N][K] B, of N (rows of B, columns of C), each slice the same block-scaled
product on a sub-block of the output.  Checked against the oracle (1e-3 * R
per element) on output rows / columns at both sides of every slice boundary,
the ends, and seeded random ones; the quantize-on-store and power-of-two
variants share the slicing and are checked on the large-A case.
"""
import numpy as np
import pytest
import torch

import fp8_precision_quant_amd as fq
import oracle
import synthetic
from gpu_util import DEV, gemm_parity, host

pytestmark = pytest.mark.gpu

K = 16384            # a row of codes is 16 KiB
BIG = (1 << 17) + 384   # 131456 rows of 16 KiB: 2.15 GB > 2^31 bytes
KB = K // 128


def _dev_codes(shape, seed):
    """Random finite E4M3 codes (never 0x7F / 0xFF), drawn on the device."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    c = torch.randint(0, 254, shape, generator=g, device=DEV, dtype=torch.uint8)
    return c + (c >= 127).to(torch.uint8)


def _dev_scales(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.rand(shape, generator=g, device=DEV, dtype=torch.float32) * 0.02 + 1e-3


def _near(edges, n, extra, seed):
    """Indices around each slice edge, both ends, and `extra` seeded ones."""
    idx = [np.arange(0, 4), np.arange(n - 4, n), synthetic.sample_rows(n, extra, seed)]
    for e in edges:
        idx.append(np.arange(e - 4, e + 4))
    idx = np.unique(np.concatenate(idx))
    return idx[(idx >= 0) & (idx < n)]


# slice edges of the library's cut for a 16 KiB row stride: 2^31 / 16384 rows
# less a two-tile margin, rounded down to 256
EDGES = [130304]


def test_large_a_sliced_over_m():
    M, N = BIG, 256
    a = _dev_codes((M, K), 1)
    sa = _dev_scales((M, KB), 2)
    b = _dev_codes((N, K), 3)
    sb = _dev_scales((N // 128, KB), 4)
    assert a.numel() >= (1 << 31)
    c = fq.fp8_gemm_blockscaled(a, sa, fq.ROW_1x128, b, sb, fq.BLOCK_128x128, fq.B_NK,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = _near(EDGES, M, 16, 5)
    ridx = torch.from_numpy(rows).to(DEV)
    a_h, sa_h = host(a.index_select(0, ridx)), host(sa.index_select(0, ridx))
    b_h, sb_h = host(b), host(sb)
    co = oracle.gemm_blockscaled(a_h, sa_h, "row", b_h, sb_h, "block", "NK")
    _, R = oracle.gemm_blockscaled(a_h, sa_h, "row", b_h, sb_h, "block", "NK", f64=True)
    gemm_parity(host(c.index_select(0, ridx)), co, R)

    # quantize-on-store over the same slices: byte-identical to the quantizer
    # applied to the fp32 result
    q, qs = fq.fp8_gemm_blockscaled_e4m3(a, sa, fq.ROW_1x128, b, sb, fq.BLOCK_128x128, fq.B_NK)
    rq, rs = fq.fp8_quant_blockwise(c, fq.ROW_1x128)
    torch.cuda.synchronize()
    assert torch.equal(q, rq)
    assert torch.equal(qs.view(torch.int32), rs.view(torch.int32))

    # power-of-two scales (E8M0 bytes 120..134), the row scales sliced as bytes
    g = torch.Generator(device=DEV)
    g.manual_seed(6)
    ea = torch.randint(120, 135, (M, KB), generator=g, device=DEV, dtype=torch.uint8)
    eb = torch.randint(120, 135, (N // 128, KB), generator=g, device=DEV, dtype=torch.uint8)
    c2 = fq.fp8_gemm_e8m0(a, ea, b, eb, fq.BLOCK_128x128, fq.B_NK, out_dtype=torch.float32)
    torch.cuda.synchronize()
    sa2 = oracle.e8m0_decode(host(ea.index_select(0, ridx)))
    sb2 = oracle.e8m0_decode(host(eb))
    co2 = oracle.gemm_blockscaled(a_h, sa2, "row", b_h, sb2, "block", "NK")
    _, R2 = oracle.gemm_blockscaled(a_h, sa2, "row", b_h, sb2, "block", "NK", f64=True)
    gemm_parity(host(c2.index_select(0, ridx)), co2, R2)


def test_large_b_sliced_over_n():
    M, N = 256, BIG
    a = _dev_codes((M, K), 11)
    sa = _dev_scales((M, KB), 12)
    b = _dev_codes((N, K), 13)
    NB = -(-N // 128)
    sb = _dev_scales((NB, KB), 14)
    assert b.numel() >= (1 << 31)
    c = fq.fp8_gemm_blockscaled(a, sa, fq.ROW_1x128, b, sb, fq.BLOCK_128x128, fq.B_NK,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    cols = _near(EDGES, N, 48, 15)
    cidx = torch.from_numpy(cols).to(DEV)
    a_h, sa_h = host(a), host(sa)
    b_h = host(b.index_select(0, cidx))                         # the B rows of the checked columns
    sb_full = host(sb)[cols // 128]                             # SB(n, kb) of those columns
    co = oracle.gemm_f32(a_h, sa_h, b_h, sb_full)
    _, R = oracle.gemm_f64(a_h, sa_h, b_h, sb_full)
    gemm_parity(host(c.index_select(1, cidx)), co, R)

    # row-scaled B (the weight-gradient mode) over the same N slices
    sbr = _dev_scales((N, KB), 16)
    c2 = fq.fp8_gemm_blockscaled(a, sa, fq.ROW_1x128, b, sbr, fq.ROW_1x128, fq.B_NK,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    sbr_h = host(sbr.index_select(0, cidx))
    co2 = oracle.gemm_f32(a_h, sa_h, b_h, sbr_h)
    _, R2 = oracle.gemm_f64(a_h, sa_h, b_h, sbr_h)
    gemm_parity(host(c2.index_select(1, cidx)), co2, R2)
