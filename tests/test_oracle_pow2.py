"""Pins of the oracle's power-of-two (E8M0) scale variant.

The pages give each block of a tensor its own scale factor in Blackwell's
micro-scaling FP8 (Introl FP8 infrastructure guide, scaling strategies and the
Blackwell section) without saying how the factor is chosen.  The reading
pinned here: s = 2^e, e the smallest integer >= -126 with amax <= 448 * 2^e,
stored as the byte e + 127; codes are E4M3(RN(x / s)).  Every expected value
below comes from exact float arithmetic in Python (``math.ldexp``, integer
comparisons), not from the oracle's own loop.
"""
import math

import numpy as np
import pytest

import oracle


def _min_exponent(amax: float) -> int:
    """The definition written out: scan e upward from -126."""
    e = -126
    while amax > 448.0 * math.ldexp(1.0, e):
        e += 1
    return e


def test_exponent_at_powers_of_two_times_448():
    # amax = 448 * 2^j exactly needs e = j; one fp32 ulp above needs j + 1;
    # one ulp below still needs j (448 * 2^(j-1) is far below it)
    for j in range(-126, 120):
        a = np.float32(math.ldexp(448.0, j))
        assert float(a) == math.ldexp(448.0, j)
        assert oracle.pow2_exponent(a) == j, j
        up = np.nextafter(a, np.float32(np.inf))
        if np.isfinite(up):
            assert oracle.pow2_exponent(up) == j + 1, j
        if j > -126:
            assert oracle.pow2_exponent(np.nextafter(a, np.float32(0))) == j, j


def test_exponent_special_values():
    assert oracle.pow2_exponent(0.0) == -126                     # zero tile
    assert oracle.pow2_exponent(np.float32(1e-45)) == -126       # smallest subnormal
    assert oracle.pow2_exponent(np.float32(2.0 ** -126)) == -126
    assert oracle.pow2_exponent(1.0) == -8                       # 1 / 2^-8 = 256 <= 448 < 512
    assert oracle.pow2_exponent(448.0) == 0
    assert oracle.pow2_exponent(449.0) == 1
    assert oracle.pow2_exponent(np.finfo(np.float32).max) == 120  # byte 247: E8M0 never overflows


def test_exponent_is_the_minimal_one_on_random_amax():
    rng = np.random.default_rng(11)
    amax = np.concatenate([
        (rng.standard_normal(4000) * 10.0 ** rng.uniform(-40, 38, 4000)).astype(np.float32),
        rng.integers(1, 0x7F7FFFFF, 4000, dtype=np.uint32).view(np.float32),  # any finite bit pattern
    ])
    for a in np.abs(amax):
        e = oracle.pow2_exponent(a)
        assert e == _min_exponent(float(a)), float(a)
        assert float(a) <= math.ldexp(448.0, e)
        assert e == -126 or float(a) > math.ldexp(448.0, e - 1)


def test_e8m0_decode_all_bytes():
    b = np.arange(256, dtype=np.uint8)
    d = oracle.e8m0_decode(b)
    for i in range(255):
        assert float(d[i]) == math.ldexp(1.0, i - 127), i
    assert np.isnan(d[255])


def _tiles(shape, tr, tc):
    R, C = shape
    for r0 in range(0, R, tr):
        for c0 in range(0, C, tc):
            yield r0 // tr, c0 // tc, slice(r0, min(r0 + tr, R)), slice(c0, min(c0 + tc, C))


@pytest.mark.parametrize("tr,tc,shape", [(1, 128, (5, 300)), (128, 128, (200, 260)), (1, 128, (3, 128))])
def test_pow2_tiles_codes_and_exponents(tr, tc, shape):
    rng = np.random.default_rng(5)
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(3e-3)
    x[rng.random(shape) < 0.002] *= 100.0         # outliers
    x[0, :] *= np.float32(2.0 ** -110)            # rows near the bottom of the E8M0 range
    if shape[1] > 128:
        x[:, 128:256] = 0.0                       # a zero tile column
    q, e = oracle.quant_tiles_pow2(x, tr, tc)
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    for ti, tj, rs, cs in _tiles(shape, tr, tc):
        t = x[rs, cs]
        amax = float(np.abs(t).max())
        ex = int(e[ti, tj]) - 127
        assert ex == _min_exponent(amax)
        s = math.ldexp(1.0, ex)
        # x / s is exact here (the smallest tile value is far above 2^-126 s),
        # so the code is the E4M3 value nearest x / s: its error is at most
        # half the E4M3 spacing around x / s, and no value saturates
        v = t.astype(np.float64) / s
        assert np.abs(v).max() <= 448.0
        got = dec[q[rs, cs]].astype(np.float64)
        ulp = np.where(np.abs(v) < 2.0 ** -6, 2.0 ** -9,
                       2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6))) - 3))
        assert np.all(np.abs(got - v) <= ulp / 2 + 0.0)
        # ties and signs: an independent nearest-even search over all codes
        cand = dec[:127].astype(np.float64)       # the non-negative finite codes
        for val, code in zip(v.ravel()[:64], q[rs, cs].ravel()[:64]):
            dist = np.abs(cand - abs(val))
            best = np.flatnonzero(dist == dist.min())
            want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
            assert (code & 0x7F) == want
            if val != 0:
                assert (code >> 7) == (val < 0)
        if amax == 0.0:
            assert ex == -126
            assert np.all((q[rs, cs] & 0x7F) == 0)


def test_pow2_scale_bounds_the_fp32_scale():
    # s_fp32 = amax / 448 <= 2^e < 2 amax / 448 (up to the fp32 rounding of
    # amax / 448) wherever the -126 floor does not bind
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((64, 1024)) * 10.0 ** rng.uniform(-6, 6, (64, 1))).astype(np.float32)
    _, s32 = oracle.quant_1x128(x)
    _, e = oracle.quant_1x128_pow2(x)
    s2 = oracle.e8m0_decode(e).astype(np.float64)
    assert np.all(s2 >= s32.astype(np.float64) * (1 - 2.0 ** -23))
    assert np.all(s2 < 2.0 * s32.astype(np.float64) * (1 + 2.0 ** -23))


def test_pow2_outlier_isolation():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((256, 512)).astype(np.float32)
    _, e0 = oracle.quant_128x128_pow2(x)
    _, r0 = oracle.quant_1x128_pow2(x)
    y = x.copy()
    y[130, 300] = 1e4                              # block (1, 2), row tile (130, 2)
    _, e1 = oracle.quant_128x128_pow2(y)
    _, r1 = oracle.quant_1x128_pow2(y)
    diff = np.argwhere(e0 != e1)
    assert diff.tolist() == [[1, 2]]
    assert np.argwhere(r0 != r1).tolist() == [[130, 2]]


def test_pow2_transpose_is_row_tiles_of_the_transpose():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((130, 260)).astype(np.float32)
    q_row, e_row, q_colT, e_colT = oracle.quant_transpose_pow2(x)
    qr, er = oracle.quant_1x128_pow2(x)
    np.testing.assert_array_equal(q_row, qr)
    np.testing.assert_array_equal(e_row, er)
    # column tile (c, j) of X covers X[128 j : 128 j + 128, c]
    for c in (0, 77, 259):
        for j in range(2):
            col = x[128 * j:128 * j + 128, c]
            assert int(e_colT[c, j]) - 127 == _min_exponent(float(np.abs(col).max()))


def test_pow2_gemm_equals_exact_dequantized_product():
    """The GEMM with decoded power-of-two scales against an fp64 matmul of
    the dequantized operands (brute force over the whole product)."""
    rng = np.random.default_rng(9)
    M, N, K = 40, 36, 300
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qa, ea = oracle.quant_1x128_pow2(x)
    qb, eb = oracle.quant_128x128_pow2(w)
    sa, sb = oracle.e8m0_decode(ea), oracle.e8m0_decode(eb)
    c = oracle.gemm_blockscaled(qa, sa, "row", qb, sb, "block", "NK")
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)
    xa = dec[qa] * np.repeat(sa.astype(np.float64), 128, axis=1)[:, :K]
    wb = dec[qb] * np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0), 128, axis=1)[:N, :K]
    ref = xa @ wb.T
    r = np.abs(xa) @ np.abs(wb).T
    assert np.all(np.abs(c - ref) <= 1e-6 * r + 1e-30)
    # and the quantized product is close to the unquantized one
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(c - exact).max() <= 0.1 * np.abs(exact).max()
