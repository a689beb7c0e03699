"""Pins for the oracle's tile quantizers.

What fixes them, other than the oracle itself:
* the quantization rule x_fp8 = Cast(x / s) (FP8-LM review, section 三, tensor
  scaling) with s = amax/448, checked through invariants that any correct
  implementation must satisfy: a tile's largest element lands on +-448, codes
  are invariant under power-of-two rescaling and odd under negation, and a
  tile built from E4M3 values plus one 448 is reproduced exactly with s = 1;
* the dequantisation error bound of a 3-mantissa-bit round-to-nearest format;
* outlier isolation, the pages' argument for per-tile scales (Ling 2.0 FP8
  blog, coarse vs fine-grained quantization): a spike changes only its own
  tile, while a per-tensor scale spreads its effect;
* a brute-force per-tile loop on tiny ragged inputs that picks, for every
  element, the nearest E4M3 value from torch's decode table.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic

TORCH_DEC = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(
    torch.float8_e4m3fn).to(torch.float64).numpy()


def _normal(shape, seed, sigma=1.0):
    return synthetic.normal_f32(shape, seed, sigma)


def _tiles(kind):
    return {"row": (1, 128), "block": (128, 128)}[kind]


@pytest.mark.parametrize("kind", ["row", "block"])
def test_scale_bits_and_max_code(kind):
    x = _normal((300, 700), 11)
    q, s = oracle.quantize(x, kind)
    tr, tc = _tiles(kind)
    assert s.shape == (-(-300 // tr), -(-700 // tc))
    for i in range(s.shape[0]):
        for j in range(s.shape[1]):
            t = x[i * tr:(i + 1) * tr, j * tc:(j + 1) * tc]
            qt = q[i * tr:(i + 1) * tr, j * tc:(j + 1) * tc]
            amax = np.float32(np.abs(t).max())
            assert s[i, j] == np.float32(amax / np.float32(448.0))
            # the tile's largest magnitude lands exactly on the largest code
            assert (qt & 0x7F).max() == 0x7E
            assert np.all((qt & 0x7F) <= 0x7E)


@pytest.mark.parametrize("kind", ["row", "block", "tensor"])
@pytest.mark.parametrize("k", [-20, -3, 5, 40])
def test_power_of_two_invariance(kind, k):
    x = _normal((260, 390), 12)
    q0, s0 = oracle.quantize(x, kind)
    q1, s1 = oracle.quantize(x * np.float32(2.0 ** k), kind)
    assert np.array_equal(q0, q1)
    assert np.array_equal(s1, s0 * np.float32(2.0 ** k))


@pytest.mark.parametrize("kind", ["row", "block", "tensor"])
def test_sign_symmetry(kind):
    x = _normal((200, 300), 13)
    q0, s0 = oracle.quantize(x, kind)
    q1, s1 = oracle.quantize(-x, kind)
    assert np.array_equal(q1, q0 ^ 0x80)
    assert np.array_equal(s0, s1)


def test_roundtrip_tile_of_codes():
    g = np.random.Generator(np.random.PCG64(14))
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    for trial in range(50):
        codes = g.choice(finite, size=128)
        codes[g.integers(128)] = 0x7E if trial % 2 else 0xFE     # one +-448
        x = oracle.e4m3_decode(codes)[None, :]
        q, s = oracle.quant_1x128(x)
        assert s[0, 0] == np.float32(1.0)
        # -0 and +0 both decode to 0; the code keeps x's sign bit
        assert np.array_equal(q[0], codes)


@pytest.mark.parametrize("kind", ["row", "block", "tensor"])
def test_dequant_error_bound(kind):
    x = synthetic.with_outliers_f32(_normal((256, 512), 15), 0.001, 100.0, 16)
    q, s = oracle.quantize(x, kind)
    tr, tc = _tiles(kind) if kind != "tensor" else x.shape
    S = np.repeat(np.repeat(s, tr, 0), tc, 1)[: x.shape[0], : x.shape[1]].astype(np.float64)
    deq = oracle.e4m3_decode(q).astype(np.float64) * S
    err = np.abs(deq - x.astype(np.float64))
    # 3 mantissa bits: relative error <= 2^-4 in the normal range; absolute
    # error <= half the subnormal spacing 2^-10 (in units of s) below 2^-6;
    # the fp32 quotient adds at most one fp32 rounding.
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * S) * (1 + 2.0 ** -20)
    assert np.all(err <= bound)


def test_outlier_isolation_row_and_block():
    x = _normal((256, 512), 17)
    i, j = 77, 300
    y = x.copy()
    y[i, j] *= np.float32(100.0)
    for kind in ["row", "block"]:
        tr, tc = _tiles(kind)
        q0, s0 = oracle.quantize(x, kind)
        q1, s1 = oracle.quantize(y, kind)
        ti, tj = i // tr, j // tc
        ds = np.argwhere(s0 != s1)
        assert ds.tolist() == [[ti, tj]]
        diff = np.argwhere(q0 != q1)
        assert diff.size > 0
        assert np.all(diff[:, 0] // tr == ti) and np.all(diff[:, 1] // tc == tj)
    # with one scale for the whole tensor the spike changes codes everywhere
    q0, s0 = oracle.quant_tensor(x)
    q1, s1 = oracle.quant_tensor(y)
    changed_rows = np.unique(np.argwhere(q0 != q1)[:, 0])
    assert changed_rows.size > 200


def test_zero_and_tiny_tiles():
    x = np.zeros((2, 256), np.float32)
    x[0, :128] = -0.0
    x[1, 128] = 1e-45                  # smallest subnormal: amax/448 underflows to 0
    x[1, 129] = -1e-45
    q, s = oracle.quant_1x128(x)
    assert np.all(s == 0)
    assert np.all(q[0, :128] == 0x80) and np.all(q[0, 128:] == 0)
    assert q[1, 128] == 0x00 and q[1, 129] == 0x80
    # a subnormal amax with a non-zero scale still quantizes its largest value to 448
    z = np.zeros((1, 128), np.float32)
    z[0, 5] = np.float32(1e-38)
    q, s = oracle.quant_1x128(z)
    assert s[0, 0] > 0 and (q[0, 5] & 0x7F) == 0x7E


def test_block_transpose_invariance():
    w = _normal((384, 260), 18)
    q, s = oracle.quant_128x128(w)
    qt, st = oracle.quant_128x128(np.ascontiguousarray(w.T))
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T)


def test_quant_transpose_columns():
    x = _normal((300, 260), 19)
    q_row, s_row, q_colT, s_colT = oracle.quant_transpose(x)
    assert q_colT.shape == (260, 300) and s_colT.shape == (260, 3)
    for c in [0, 1, 129, 259]:
        for i in range(3):
            col = x[i * 128:(i + 1) * 128, c]
            assert s_colT[c, i] == np.float32(np.abs(col).max() / np.float32(448.0))
    qr, sr = oracle.quant_1x128(x)
    assert np.array_equal(qr, q_row) and np.array_equal(sr, s_row)


def _bruteforce_tile_quant(x, tr, tc):
    """Per-tile loop; each code chosen as the nearest E4M3 value (torch table)."""
    finite = [c for c in range(128) if c != 0x7F]
    mags = TORCH_DEC[finite]
    R, C = x.shape
    q = np.zeros((R, C), np.uint8)
    s = np.zeros((-(-R // tr), -(-C // tc)), np.float32)
    for ti in range(s.shape[0]):
        for tj in range(s.shape[1]):
            t = x[ti * tr:(ti + 1) * tr, tj * tc:(tj + 1) * tc]
            amax = np.float32(0)
            for v in t.reshape(-1):
                amax = max(amax, np.float32(abs(v)))
            sc = np.float32(amax / np.float32(448))
            s[ti, tj] = sc
            for (r, c), v in np.ndenumerate(t):
                sign = 0x80 if np.signbit(v) else 0
                if sc == 0:
                    code = 0
                else:
                    a = abs(float(np.float32(v / sc)))
                    if a > 448:
                        code = 0x7E
                    else:
                        d = np.abs(mags - a)
                        best = np.nonzero(d == d.min())[0]
                        cands = [finite[b] for b in best]
                        code = [cc for cc in cands if cc % 2 == 0][0] if len(cands) > 1 else cands[0]
                q[ti * tr + r, tj * tc + c] = sign | code
    return q, s


@pytest.mark.parametrize("shape,tr,tc", [((3, 300), 1, 128), ((130, 140), 128, 128)])
def test_bruteforce_tiny_ragged(shape, tr, tc):
    g = np.random.Generator(np.random.PCG64(20))
    x = (g.standard_normal(shape) * np.exp(g.standard_normal(shape) * 3)).astype(np.float32)
    x[0, 0] = -0.0
    qo, so = oracle.quant_tiles(x, tr, tc)
    qb, sb = _bruteforce_tile_quant(x, tr, tc)
    assert np.array_equal(so, sb)
    assert np.array_equal(qo, qb)


def test_underflow_fraction():
    x = np.ones((1, 128), np.float32)
    x[0, :10] = 1e-6               # x/s = 4.5e-4 < 2^-10 (half the smallest subnormal)
    x[0, 10:20] = 0.0              # zeros do not count
    q, s = oracle.quant_1x128(x)
    assert oracle.underflow_fraction(x, q) == pytest.approx(10 / 118)
