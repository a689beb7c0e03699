"""GPU parity of the grouped (MoE expert) GEMMs: fp8_grouped_gemm (forward),
fp8_grouped_gemm_e4m3 (the forward stored as E4M3 codes with 1x128 scales),
fp8_grouped_gemm_dgrad and fp8_grouped_gemm_wgrad (backward).

Groups are padded with zero rows to multiples of 128 (Ling 2.0 FP8 blog,
"FP8 padding routing map": padded rows do not change the result).  Bar as in
the dense GEMM (1e-3 * R per element, exact zeros where R == 0), plus: every
group equals the dense GEMM with that expert's weights, pad rows are exactly
zero, empty groups are skipped, and rows past the last group are untouched.
The backward: dgrad reads each expert's weight as stored and must equal the
oracle's per-group dgrad; wgrad sums each expert's tokens only (empty groups
give exactly 0) from the transposed re-quantization of dY and X.  The
quantized forward must be byte for byte the GPU quantizer's output on the
fp32 forward's rows [0, off[G]), leave the rest untouched, and be a valid
quantization of the oracle's result (as for the dense quantize-on-store).
Workload: 8192 tokens, hidden 2048, 128 experts of intermediate 768, top-8
Zipf(1.1) routing, gate/up (N=1536, K=2048) and down (N=2048, K=768).
"""
import numpy as np
import pytest
import torch

import fp8_precision_quant_amd as fq
import oracle
import synthetic
from gpu_util import DEV, bf16_parity, gemm_parity, host, to_dev

pytestmark = pytest.mark.gpu

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _codes(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).choice(FINITE, size=shape)


def _scales(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return (np.exp(g.standard_normal(shape)) * 0.01).astype(np.float32)


def _run(a, sa, off, b, sb, out=torch.float32, c=None):
    c = fq.fp8_grouped_gemm(to_dev(a), to_dev(sa), to_dev(off.astype(np.int32)), to_dev(b),
                            to_dev(sb), out_dtype=out, c=c)
    torch.cuda.synchronize()
    return c


# K = 400 takes the kernel that masks a partial last chunk; K = 384 (whole
# chunks) the four-wave kernel
@pytest.mark.parametrize("K", [400, 384])
def test_small_groups_with_empty_and_ragged(K):
    counts = [100, 0, 260, 1, 0, 128]
    G, N = len(counts), 300
    KB = -(-K // 128)
    off = np.concatenate([[0], np.cumsum([-(-c // 128) * 128 for c in counts])])
    M = int(off[-1])
    A = np.zeros((M, K), np.uint8)
    sa = np.zeros((M, KB), np.float32)
    for e, cnt in enumerate(counts):
        A[off[e]:off[e] + cnt] = _codes((cnt, K), 10 + e)
        sa[off[e]:off[e] + cnt] = _scales((cnt, KB), 20 + e)
    B = _codes((G, N, K), 30)
    sb = _scales((G, 3, KB), 31)
    c = host(_run(A, sa, off, B, sb))
    co = oracle.grouped_gemm(A, sa, off, B, sb)
    _, R = oracle.grouped_gemm(A, sa, off, B, sb, f64=True)
    gemm_parity(c, co, R)
    for e, cnt in enumerate(counts):
        assert np.all(c[off[e] + cnt:off[e + 1]] == 0)


def test_rows_past_last_group_untouched():
    G, N, K = 2, 256, 256
    off = np.array([0, 128, 256])
    M_pad = 512                          # last 256 rows belong to no group
    A = _codes((M_pad, K), 40)
    sa = _scales((M_pad, 2), 41)
    B = _codes((G, N, K), 42)
    sb = _scales((G, 2, 2), 43)
    c = torch.full((M_pad, N), -9.0, dtype=torch.float32, device=DEV)
    _run(A, sa, off, B, sb, c=c)
    ch = host(c)
    assert np.all(ch[256:] == -9.0)
    co = oracle.grouped_gemm(A[:256], sa[:256], off, B, sb)
    _, R = oracle.grouped_gemm(A[:256], sa[:256], off, B, sb, f64=True)
    gemm_parity(ch[:256], co, R)


@pytest.fixture(scope="module")
def moe_inputs():
    m = synthetic.moe()
    qa, sa = oracle.quant_1x128(synthetic.bf16_to_f32(m.a_gate_up))
    qa2, sa2 = oracle.quant_1x128(synthetic.bf16_to_f32(m.a_down))
    G = m.w_gate_up.shape[0]
    qgu = np.empty(m.w_gate_up.shape, np.uint8)
    sgu = np.empty((G, 12, 16), np.float32)
    qd = np.empty(m.w_down.shape, np.uint8)
    sd = np.empty((G, 16, 6), np.float32)
    for e in range(G):
        qgu[e], sgu[e] = oracle.quant_128x128(synthetic.bf16_to_f32(m.w_gate_up[e]))
        qd[e], sd[e] = oracle.quant_128x128(synthetic.bf16_to_f32(m.w_down[e]))
    return m, (qa, sa, qgu, sgu), (qa2, sa2, qd, sd)


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_moe_full_size_row_per_tile(moe_inputs, which):
    m, gu, dn = moe_inputs
    qa, sa, qb, sb = gu if which == "gate_up" else dn
    off = m.offsets.astype(np.int64)
    c32 = host(_run(qa, sa, off, qb, sb))
    cb = host(_run(qa, sa, off, qb, sb, out=torch.bfloat16))
    # one seeded row in every 128-row tile (every group, pad rows included),
    # plus the first rows of the most and least loaded experts
    big = int(np.argmax(m.counts))
    small = int(np.argmin(m.counts))
    rows = np.concatenate([np.arange(off[big], off[big] + 6), np.arange(off[small], off[small] + 4),
                           synthetic.rows_per_tile(qa.shape[0], 404)])
    rows = np.unique(rows)
    co = oracle.grouped_gemm(qa, sa, off, qb, sb, rows=rows)
    _, R = oracle.grouped_gemm(qa, sa, off, qb, sb, rows=rows, f64=True)
    gemm_parity(c32[rows], co, R)
    bf16_parity(cb[rows], c32[rows], co, R, oracle.f32_to_bf16_bits(c32[rows]))
    pad = m.token_index < 0
    assert np.all(c32[pad] == 0)


def _groups(counts):
    return np.concatenate([[0], np.cumsum([-(-c // 128) * 128 for c in counts])]).astype(np.int64)


def _run_dgrad(a, sa, off, w, sw, out=torch.float32, c=None):
    c = fq.fp8_grouped_gemm_dgrad(to_dev(a), to_dev(sa), to_dev(off.astype(np.int32)), to_dev(w),
                                  to_dev(sw), out_dtype=out, c=c)
    torch.cuda.synchronize()
    return c


def _run_wgrad(at, sat, bt, sbt, off, c=None):
    c = fq.fp8_grouped_gemm_wgrad(to_dev(at), to_dev(sat), to_dev(bt), to_dev(sbt),
                                  to_dev(off.astype(np.int32)), c=c)
    torch.cuda.synchronize()
    return c


# contraction N = 300 (a partial last chunk) takes the eight-wave kernel,
# N = 384 the four-wave kernel's transposing reads; K = 400 leaves a ragged
# last column tile either way
@pytest.mark.parametrize("N", [300, 384])
def test_dgrad_small_groups_with_empty_and_ragged(N):
    counts = [100, 0, 260, 1, 0, 128]
    G, K = len(counts), 400
    NB = -(-N // 128)
    off = _groups(counts)
    M = int(off[-1])
    A = np.zeros((M, N), np.uint8)
    sa = np.zeros((M, NB), np.float32)
    for e, cnt in enumerate(counts):
        A[off[e]:off[e] + cnt] = _codes((cnt, N), 110 + e)
        sa[off[e]:off[e] + cnt] = _scales((cnt, NB), 120 + e)
    W = _codes((G, N, K), 130)
    sw = _scales((G, NB, 4), 131)
    c = host(_run_dgrad(A, sa, off, W, sw))
    co = oracle.grouped_gemm_dgrad(A, sa, off, W, sw)
    _, R = oracle.grouped_gemm_dgrad(A, sa, off, W, sw, f64=True)
    gemm_parity(c, co, R)
    cb = host(_run_dgrad(A, sa, off, W, sw, out=torch.bfloat16))
    bf16_parity(cb, c, co, R, oracle.f32_to_bf16_bits(c))
    for e, cnt in enumerate(counts):
        assert np.all(c[off[e] + cnt:off[e + 1]] == 0)


def test_dgrad_rows_past_last_group_untouched():
    G, N, K = 2, 256, 320
    off = np.array([0, 128, 256])
    M_pad = 384                              # the last 128 rows belong to no group
    A = _codes((M_pad, N), 140)
    sa = _scales((M_pad, 2), 141)
    W = _codes((G, N, K), 142)
    sw = _scales((G, 2, 3), 143)
    c = torch.full((M_pad, K), -9.0, dtype=torch.float32, device=DEV)
    _run_dgrad(A, sa, off, W, sw, c=c)
    ch = host(c)
    assert np.all(ch[256:] == -9.0)
    co = oracle.grouped_gemm_dgrad(A[:256], sa[:256], off, W, sw)
    _, R = oracle.grouped_gemm_dgrad(A[:256], sa[:256], off, W, sw, f64=True)
    gemm_parity(ch[:256], co, R)


def test_wgrad_small_groups_with_empty_and_ragged():
    counts = [200, 0, 128, 60, 1, 0]
    G, N, K = len(counts), 150, 260
    off = _groups(counts)
    M = int(off[-1])
    g = np.random.Generator(np.random.PCG64(150))
    dy = g.standard_normal((M, N)).astype(np.float32)
    x = g.standard_normal((M, K)).astype(np.float32) * 3
    for e, cnt in enumerate(counts):
        dy[off[e] + cnt:off[e + 1]] = 0
        x[off[e] + cnt:off[e + 1]] = 0
    at, sat = oracle.quant_1x128(np.ascontiguousarray(dy.T))
    bt, sbt = oracle.quant_1x128(np.ascontiguousarray(x.T))
    # output in a wider buffer: columns past K must stay untouched
    buf = torch.full((G, N, 272), -7.0, dtype=torch.float32, device=DEV)
    _run_wgrad(at, sat, bt, sbt, off, c=buf[:, :, :K])
    hb = host(buf)
    assert np.all(hb[:, :, K:] == -7.0)
    co = oracle.grouped_gemm_wgrad(at, sat, bt, sbt, off)
    _, R = oracle.grouped_gemm_wgrad(at, sat, bt, sbt, off, f64=True)
    for e in range(G):
        gemm_parity(hb[e, :, :K], co[e], R[e])
        if counts[e] == 0:
            assert np.all(hb[e, :, :K] == 0)


def test_wgrad_one_group_holds_every_token():
    # a single non-empty group: one XCD computes, every workgroup zero-fills
    counts = [0, 0, 390, 0]
    G, N, K = len(counts), 256, 512
    off = _groups(counts)
    M = int(off[-1])
    g = np.random.Generator(np.random.PCG64(151))
    dy = g.standard_normal((M, N)).astype(np.float32)
    x = g.standard_normal((M, K)).astype(np.float32)
    dy[off[2] + counts[2]:] = 0
    x[off[2] + counts[2]:] = 0
    at, sat = oracle.quant_1x128(np.ascontiguousarray(dy.T))
    bt, sbt = oracle.quant_1x128(np.ascontiguousarray(x.T))
    buf = torch.full((G, N, K), -7.0, dtype=torch.float32, device=DEV)
    hb = host(_run_wgrad(at, sat, bt, sbt, off, c=buf))
    co = oracle.grouped_gemm_wgrad(at, sat, bt, sbt, off)
    _, R = oracle.grouped_gemm_wgrad(at, sat, bt, sbt, off, f64=True)
    gemm_parity(hb[2], co[2], R[2])
    for e in (0, 1, 3):
        assert np.all(hb[e] == 0)


def test_wgrad_without_tokens_is_zero():
    G, N, K = 3, 130, 300
    off = np.zeros(G + 1, np.int64)
    at, sat = np.zeros((N, 0), np.uint8), np.zeros((N, 0), np.float32)
    bt, sbt = np.zeros((K, 0), np.uint8), np.zeros((K, 0), np.float32)
    buf = torch.full((G, N, K), -7.0, dtype=torch.float32, device=DEV)
    assert np.all(host(_run_wgrad(at, sat, bt, sbt, off, c=buf)) == 0)


@pytest.fixture(scope="module")
def moe_backward(moe_inputs):
    m, gu, dn = moe_inputs
    dgu, dd = synthetic.moe_backward_dy(m)
    dgu32, dd32 = synthetic.bf16_to_f32(dgu), synthetic.bf16_to_f32(dd)
    return m, gu, dn, dgu32, dd32


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_moe_dgrad_full_size_row_per_tile(moe_backward, which):
    m, gu, dn, dgu, dd = moe_backward
    _, _, qw, sw = gu if which == "gate_up" else dn
    qdy, sdy = oracle.quant_1x128(dgu if which == "gate_up" else dd)
    off = m.offsets.astype(np.int64)
    c32 = host(_run_dgrad(qdy, sdy, off, qw, sw))
    big, small = int(np.argmax(m.counts)), int(np.argmin(m.counts))
    rows = np.unique(np.concatenate([np.arange(off[big], off[big] + 6), np.arange(off[small], off[small] + 4),
                                     synthetic.rows_per_tile(qdy.shape[0], 407)]))
    co = oracle.grouped_gemm_dgrad(qdy, sdy, off, qw, sw, rows=rows)
    _, R = oracle.grouped_gemm_dgrad(qdy, sdy, off, qw, sw, rows=rows, f64=True)
    gemm_parity(c32[rows], co, R)
    assert np.all(c32[m.token_index < 0] == 0)


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_moe_wgrad_full_size_row_per_tile(moe_backward, which):
    # dW_e = dY_e^T X_e over each expert's tokens; X is the expert GEMM's input
    m, gu, dn, dgu, dd = moe_backward
    dy = dgu if which == "gate_up" else dd
    xin = synthetic.bf16_to_f32(m.a_gate_up if which == "gate_up" else m.a_down)
    at, sat = oracle.quant_1x128(np.ascontiguousarray(dy.T))
    bt, sbt = oracle.quant_1x128(np.ascontiguousarray(xin.T))
    off = m.offsets.astype(np.int64)
    c = host(_run_wgrad(at, sat, bt, sbt, off))
    rows = synthetic.rows_per_tile(at.shape[0], 408)
    co = oracle.grouped_gemm_wgrad(at, sat, bt, sbt, off, rows=rows)
    _, R = oracle.grouped_gemm_wgrad(at, sat, bt, sbt, off, rows=rows, f64=True)
    for e in range(c.shape[0]):
        gemm_parity(c[e][rows], co[e], R[e])


def _run_e4m3(a, sa, off, b, sb, q=None, s=None):
    q, s = fq.fp8_grouped_gemm_e4m3(to_dev(a), to_dev(sa), to_dev(off.astype(np.int32)), to_dev(b),
                                    to_dev(sb), q=q, s=s)
    torch.cuda.synchronize()
    return q, s


def _e4m3_matches_quantized_fp32(a, sa, off, b, sb):
    """Codes and scales of the quantized grouped forward against the GPU
    quantizer run on the fp32 grouped forward, rows [0, off[G]): byte equal."""
    q, s = _run_e4m3(a, sa, off, b, sb)
    c = _run(a, sa, off, b, sb)
    used = int(off[-1])
    rq, rs = fq.fp8_quant_blockwise(c[:used], fq.ROW_1x128)
    torch.cuda.synchronize()
    assert torch.equal(q[:used], rq)
    assert torch.equal(s[:used].view(torch.int32), rs.view(torch.int32))
    return host(q), host(s)


def _e4m3_valid(q, s, co, R):
    """A valid 1x128 quantization of the oracle's result co (rows of q, s):
    each tile's scale within the GEMM tolerance of its amax / 448, each
    dequantized code within half an E4M3 step of co plus that tolerance."""
    co = co.astype(np.float64)
    n, N = co.shape
    NB = -(-N // 128)
    pad = NB * 128 - N
    amax_o = np.abs(np.pad(co, ((0, 0), (0, pad)))).reshape(n, NB, 128).max(axis=2)
    tol_t = 1e-3 * np.pad(R, ((0, 0), (0, pad))).reshape(n, NB, 128).max(axis=2)
    assert np.all(np.abs(s[:, :NB].astype(np.float64) * 448 - amax_o) <= tol_t * 1.0001 + 1e-30)
    s_full = np.repeat(s[:, :NB].astype(np.float64), 128, axis=1)[:, :N]
    deq = oracle.e4m3_decode(q[:, :N]).astype(np.float64) * s_full
    half_step = np.maximum(np.abs(co) * 2.0 ** -4, s_full * 2.0 ** -10)
    assert np.all(np.abs(deq - co) <= half_step * 1.0001 + 1e-3 * R * 2 + 1e-30)


# N = 300 leaves a ragged last scale tile; K = 384 and 128 are whole chunks
@pytest.mark.parametrize("N,K", [(300, 384), (256, 128)])
def test_e4m3_small_groups_with_empty_and_ragged(N, K):
    counts = [100, 0, 260, 1, 0, 128]
    G, KB = len(counts), K // 128
    off = _groups(counts)
    M = int(off[-1])
    A = np.zeros((M, K), np.uint8)
    sa = np.zeros((M, KB), np.float32)
    for e, cnt in enumerate(counts):
        A[off[e]:off[e] + cnt] = _codes((cnt, K), 210 + e)
        sa[off[e]:off[e] + cnt] = _scales((cnt, KB), 220 + e)
    B = _codes((G, N, K), 230)
    sb = _scales((G, -(-N // 128), KB), 231)
    q, s = _e4m3_matches_quantized_fp32(A, sa, off, B, sb)
    co = oracle.grouped_gemm(A, sa, off, B, sb)
    _, R = oracle.grouped_gemm(A, sa, off, B, sb, f64=True)
    _e4m3_valid(q, s, co, R)
    for e, cnt in enumerate(counts):                 # pad rows: zero codes, zero scales
        assert np.all(q[off[e] + cnt:off[e + 1]] == 0)
        assert np.all(s[off[e] + cnt:off[e + 1]] == 0)


def test_e4m3_rows_past_last_group_and_columns_past_n_untouched():
    G, N, K = 2, 200, 256
    off = np.array([0, 128, 256])
    M_pad = 512                              # the last 256 rows belong to no group
    A = _codes((M_pad, K), 240)
    sa = _scales((M_pad, 2), 241)
    B = _codes((G, N, K), 242)
    sb = _scales((G, 2, 2), 243)
    qbuf = torch.full((M_pad, 224), 0x5A, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((M_pad, 3), -9.0, dtype=torch.float32, device=DEV)
    q, s = _run_e4m3(A, sa, off, B, sb, q=qbuf[:, :N], s=sbuf[:, :2])
    qh, sh = host(qbuf), host(sbuf)
    assert np.all(qh[256:] == 0x5A) and np.all(qh[:, N:] == 0x5A)
    assert np.all(sh[256:] == -9.0) and np.all(sh[:, 2:] == -9.0)
    co = oracle.grouped_gemm(A[:256], sa[:256], off, B, sb)
    _, R = oracle.grouped_gemm(A[:256], sa[:256], off, B, sb, f64=True)
    _e4m3_valid(qh[:256, :N], sh[:256, :2], co, R)


def test_e4m3_rejects_ragged_k():
    counts = [128]
    off = _groups(counts)
    A, sa = _codes((128, 200), 250), _scales((128, 2), 251)
    B, sb = _codes((1, 128, 200), 252), _scales((1, 1, 2), 253)
    with pytest.raises(fq.Fp8qError, match="UNSUPPORTED"):
        _run_e4m3(A, sa, off, B, sb)


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_moe_e4m3_full_size(moe_inputs, which):
    """Both MoE expert GEMMs at full size (the launches the MoE leg of the
    bench times): codes and scales byte-identical over every grouped row to
    the GPU quantizer on the fp32 grouped forward; on one row of every
    128-row tile, a valid quantization of the oracle's result."""
    m, gu, dn = moe_inputs
    qa, sa, qb, sb = gu if which == "gate_up" else dn
    off = m.offsets.astype(np.int64)
    q, s = _e4m3_matches_quantized_fp32(qa, sa, off, qb, sb)
    rows = synthetic.rows_per_tile(qa.shape[0], 409)
    co = oracle.grouped_gemm(qa, sa, off, qb, sb, rows=rows)
    _, R = oracle.grouped_gemm(qa, sa, off, qb, sb, rows=rows, f64=True)
    _e4m3_valid(q[rows], s[rows], co, R)
    pad = m.token_index < 0
    assert np.all(q[pad] == 0) and np.all(s[pad] == 0)
