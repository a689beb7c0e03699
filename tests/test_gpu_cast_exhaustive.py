"""Exhaustive GPU checks of the quantizers' quotient and E4M3 cast.

The rule is code = E4M3(RN_fp32(x / s)) with s = amax / 448 (FP8-LM review,
section 三, tensor scaling; E4M3 range +-448: "FP8-RL" article, section 一).
The kernels do not divide per element: for s >= 2^-90 they form the quotient
from the tile's correctly rounded reciprocal with one FMA correction
(Markstein), below that the IEEE quotient (or, in the quantize + transpose
kernel, the corrected reciprocal of s 2^64 applied to x 2^64), and they cast
with the hardware's packed fp32 -> fp8 conversion, clamping to +-448 first
only where a quotient can exceed 448 (1 + 2^-23), i.e. where some tile of
reach has a subnormal scale.  Those steps are checked here bit for bit
against the oracle, which divides and encodes by the definition:

(a) scale sweep: tiles whose one fixed element +-A sets amax (so s = A / 448),
    filled with every finite bf16 value x with A 2^-21 <= |x| <= A (every x
    whose quotient can reach a non-zero code, and the first ones that cannot)
    plus random fp32 values in the same window:
      - every positive finite bf16 A (bf16 inputs: 32639 scales, subnormal
        and zero s included);
      - 16384 fp32 A spread log-uniformly over the whole fp32 range, and the
        A that give s = 2^-90 and its two neighbours, the smallest normal s
        and the largest s (fp32 inputs);
(b) unit scale: tiles holding one +-448 (s = 1 exactly) filled with every
    fp32 bit pattern of magnitude <= 448 (2.28e9 values), so the clamp and
    the conversion are compared with the oracle's encoder on every value
    they can receive from a tile.

(c) quotients above 448: amax values A whose own quotient RN(A / RN(A/448))
    is 448 + 2^-15 (RN(A/448) rounded down; about one amax in twelve), which
    the unclamped cast must still map to the largest finite code.

Each data set goes through every kernel that quantizes with fp32 scales: the
1x128 row kernel, the 128x128 block kernel and the per-tensor kernels where
their tiles see the same scales, the quantize + transpose kernel's row
path (on X) and its column path (on X^T, whose column tiles are X's rows).
"""
import numpy as np
import pytest
import torch

import fp8_precision_quant_amd as fq
import oracle
import synthetic
from gpu_util import DEV, host

pytestmark = pytest.mark.gpu

# every non-negative finite bf16 bit pattern, in increasing order of value
_POS_BITS = np.arange(0x7F80, dtype=np.uint16)
_POS_F32 = synthetic.bf16_to_f32(_POS_BITS)
_LOW = 2.0 ** -21    # |x| >= A 2^-21 covers every quotient >= 2^-12 (below half the least code)


def _bf16_window(lo: float, hi: float) -> np.ndarray:
    """Every bf16 value (as fp32) with lo <= |v| <= hi, both signs."""
    a = np.searchsorted(_POS_F32, np.float32(lo), "left")
    b = np.searchsorted(_POS_F32, np.float32(hi), "right")
    p = _POS_F32[a:b]
    return np.concatenate([p, -p])


def _f32_window(lo: float, hi: float, n: int, g) -> np.ndarray:
    """n random fp32 values with lo <= |v| <= hi, uniform in the bit pattern."""
    lb = int(np.float32(lo).view(np.uint32))
    hb = int(np.float32(hi).view(np.uint32))
    bits = g.integers(lb, hb + 1, size=n, dtype=np.uint64).astype(np.uint32)
    bits |= (g.integers(0, 2, size=n, dtype=np.uint32) << 31)
    return bits.view(np.float32)


def _tiles(amaxes, frees) -> np.ndarray:
    """Tiles [T, 128]: for each (A, F) ceil(|F| / 127) tiles, column 0 holding
    +A or -A (alternating from tile to tile) and columns 1..127 the values F
    (zero-padded)."""
    out = []
    for A, F in zip(amaxes, frees):
        n = max(1, -(-F.size // 127))
        t = np.zeros((n, 128), np.float32)
        t[0::2, 0] = np.float32(A)
        t[1::2, 0] = -np.float32(A)
        flat = np.zeros(n * 127, np.float32)
        flat[:F.size] = F
        t[:, 1:] = flat.reshape(n, 127)
        out.append(t)
    return np.concatenate(out)


def _dev(x: np.ndarray, bf16: bool) -> torch.Tensor:
    """[T, 128] host tiles -> device (fp32, or bf16: the values are bf16-exact)."""
    t = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    return t.to(torch.bfloat16) if bf16 else t


def _transposed(xd: torch.Tensor) -> torch.Tensor:
    """X^T [128, T] on the device with a 16-byte aligned row stride."""
    T = xd.shape[0]
    per = 16 // xd.element_size()
    buf = torch.empty((128, -(-T // per) * per), dtype=xd.dtype, device=DEV)
    view = buf[:, :T]
    view.copy_(xd.t())
    return view


def _same(name, got, want):
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s differs at %d places, first %s (gpu %s, oracle %s)" % (
        name, len(bad), bad[0].tolist(), got[tuple(bad[0])], want[tuple(bad[0])])


def _check_rows(x: np.ndarray, bf16: bool, block_and_tensor: bool = False) -> np.ndarray:
    """Every fp32-scale kernel on the tiles x[T, 128] against the oracle's
    1x128 quantization; returns the oracle scales."""
    qo, so = oracle.quant_1x128(x)
    xd = _dev(x, bf16)
    q, s = fq.fp8_quant_blockwise(xd, fq.ROW_1x128)
    qr, sr, _, _ = fq.fp8_quant_transpose(xd, cols_out=False)
    _, _, qc, sc = fq.fp8_quant_transpose(_transposed(xd), rows_out=False)
    torch.cuda.synchronize()
    _same("row kernel codes", host(q), qo)
    _same("row kernel scales", host(s), so)
    _same("quant+transpose row codes", host(qr), qo)
    _same("quant+transpose row scales", host(sr), so)
    _same("quant+transpose column codes", host(qc), qo)
    _same("quant+transpose column scales", host(sc), so)
    if block_and_tensor:
        # every tile has the same scale, so blocks and the whole tensor do too
        assert np.all(so.view(np.uint32) == so.view(np.uint32)[0, 0])
        qb, sb = fq.fp8_quant_blockwise(xd, fq.BLOCK_128x128)
        qt, st = fq.fp8_quant_blockwise(xd, fq.TENSOR)
        torch.cuda.synchronize()
        _same("block kernel codes", host(qb), qo)
        assert np.all(host(sb).view(np.uint32) == so.view(np.uint32)[0, 0])
        _same("tensor kernel codes", host(qt), qo)
        assert host(st).view(np.uint32)[0, 0] == so.view(np.uint32)[0, 0]
    return so


def _scale_for(s_target: np.float32) -> np.float32:
    """An fp32 A with RN(A / 448) == s_target (searched around 448 s)."""
    a0 = np.float32(np.float64(s_target) * 448.0).view(np.uint32)
    for d in range(-64, 65):
        A = (a0 + np.uint32(d) if d >= 0 else a0 - np.uint32(-d)).view(np.float32)
        if np.float32(A) / np.float32(448.0) == s_target:
            return np.float32(A)
    raise AssertionError("no amax for scale %r" % s_target)


def test_scale_sweep_every_bf16_amax():
    """Every positive finite bf16 amax (32639 scales) x every bf16 x in its
    window, through the bf16-input kernels."""
    amaxes = _POS_F32[1:]
    half = amaxes.size // 2
    for part in (amaxes[:half], amaxes[half:]):
        frees = [_bf16_window(A * _LOW, A) for A in part]
        x = _tiles(part, frees)
        assert x.shape[0] > (1 << 19)   # also the row kernel's two-tiles-per-row form
        _check_rows(x, bf16=True)


def test_scale_sweep_fp32_amax():
    """16384 log-uniform fp32 amax values plus the division-path boundary
    (s = 2^-90 and one ulp either side), the least normal s and the largest
    s, each with every bf16 x and 508 random fp32 x of its window."""
    g = synthetic.rng(71)
    bits = np.sort(g.integers(1, 0x7F800000, size=16384, dtype=np.uint64).astype(np.uint32))
    s90 = np.float32(2.0 ** -90)
    special = [_scale_for(s90), _scale_for(np.nextafter(s90, np.float32(0))),
               _scale_for(np.nextafter(s90, np.float32(1))), _scale_for(np.float32(2.0 ** -126)),
               np.float32(np.finfo(np.float32).max), np.float32(448.0)]
    amaxes = np.concatenate([np.array(special, np.float32), bits.view(np.float32)])
    seen = set()
    for c0 in range(0, amaxes.size, 2048):
        part = amaxes[c0:c0 + 2048]
        frees = [np.concatenate([_bf16_window(A * _LOW, A), _f32_window(A * _LOW, A, 508, g)])
                 for A in part]
        so = _check_rows(_tiles(part, frees), bf16=False)
        seen.update(so.view(np.uint32).reshape(-1).tolist())
    # the boundary cases were hit: s = 2^-90 and both neighbours, a subnormal s
    u90 = int(s90.view(np.uint32))
    assert {u90 - 1, u90, u90 + 1} <= seen
    assert any(0 < u < 0x00800000 for u in seen)


def test_scale_sweep_blocks():
    """The 128x128 block and per-tensor kernels on a subset of the fp32 scale
    sweep: one block per amax (A at a seeded position) filled with its window."""
    g = synthetic.rng(72)
    bits = np.sort(g.integers(1, 0x7F800000, size=1024, dtype=np.uint64).astype(np.uint32))
    amaxes = np.concatenate([np.array([_scale_for(np.float32(2.0 ** -90))], np.float32), bits.view(np.float32)])
    blocks = []
    for i, A in enumerate(amaxes):
        F = np.concatenate([_bf16_window(A * _LOW, A), _f32_window(A * _LOW, A, 1000, g)])
        blk = np.zeros(128 * 128, np.float32)
        n = min(F.size, blk.size - 1)
        blk[:n] = F[:n]
        blk[-1] = A if i % 2 else -A
        blocks.append(g.permutation(blk).reshape(128, 128))
    # a column of blocks: block (i, 0) is amax i
    x = np.concatenate(blocks)
    qo, so = oracle.quant_128x128(x)
    q, s = fq.fp8_quant_blockwise(_dev(x, False), fq.BLOCK_128x128)
    torch.cuda.synchronize()
    _same("block kernel codes", host(q), qo)
    _same("block kernel scales", host(s), so)
    # per-tensor: one tensor per amax, 32 of them
    for i in range(0, amaxes.size, amaxes.size // 32):
        xb = np.ascontiguousarray(blocks[i])
        qo, so = oracle.quant_tensor(xb)
        qt, st = fq.fp8_quant_blockwise(_dev(xb, False), fq.TENSOR)
        torch.cuda.synchronize()
        _same("tensor kernel codes", host(qt), qo)
        _same("tensor kernel scale", host(st), so)


def test_unit_scale_every_fp32_value_up_to_448():
    """s = 1 tiles (one +-448 each) over every fp32 bit pattern with
    |v| <= 448, both signs: 2^23 magnitudes per chunk, 136 chunks."""
    top = int(np.float32(448.0).view(np.uint32))   # 0x43E00000
    step = 1 << 23
    n_chunks = 0
    for a in range(0, top + 1, step):
        mags = np.arange(a, min(a + step, top + 1), dtype=np.uint32)
        vals = np.concatenate([mags, mags | np.uint32(0x80000000)]).view(np.float32)
        so = _check_rows(_tiles([np.float32(448.0)], [vals]), bf16=False, block_and_tensor=True)
        assert so.view(np.uint32)[0, 0] == np.float32(1.0).view(np.uint32)
        n_chunks += 1
    assert n_chunks == 136


def _over_448(amaxes: np.ndarray) -> np.ndarray:
    """The amax values whose quotient RN(A / RN(A / 448)) exceeds 448."""
    A = amaxes.astype(np.float32)
    return A[(A / (A / np.float32(448.0))) > np.float32(448.0)]


def test_quotient_above_448_casts_to_largest_code():
    """(c): every bf16 amax with a normal scale whose own quotient rounds to
    448 + 2^-15, and 4096 such fp32 amax values, each in a tile with its bf16
    window, through the row, quantize + transpose (both paths) and 128x128
    kernels; the amax element's code is 0x7E (0xFE for -A)."""
    lo = np.float32(448.0 * 2.0 ** -126)
    bf = _over_448(_POS_F32[_POS_F32 >= lo])
    assert bf.size > 2000
    g = synthetic.rng(73)
    bits = g.integers(int(lo.view(np.uint32)), 0x7F000000, size=65536, dtype=np.uint64).astype(np.uint32)
    f32 = _over_448(bits.view(np.float32))[:4096]
    assert f32.size == 4096
    assert np.all(f32 / (f32 / np.float32(448.0)) == np.float32(448.0 + 2.0 ** -15))
    for amaxes, bf16 in ((bf, True), (f32, False)):
        frees = [_bf16_window(A * np.float32(0.5), A) for A in amaxes]
        x = _tiles(amaxes, frees)
        _check_rows(x, bf16=bf16)
        qo, _ = oracle.quant_1x128(x)
        first = np.concatenate([[0], np.cumsum([max(1, -(-F.size // 127)) for F in frees])[:-1]])
        assert np.all(qo[first, 0] == 0x7E)
    # 128x128 blocks: amax A at a seeded position of a block of its window
    blocks = []
    for i, A in enumerate(bf[:512]):
        F = _bf16_window(A * np.float32(0.5), A)
        blk = np.zeros(128 * 128, np.float32)
        n = min(F.size, blk.size - 1)
        blk[:n] = F[:n]
        blk[-1] = A if i % 2 else -A
        blocks.append(g.permutation(blk).reshape(128, 128))
    x = np.concatenate(blocks)
    qo, so = oracle.quant_128x128(x)
    q, s = fq.fp8_quant_blockwise(_dev(x, True), fq.BLOCK_128x128)
    torch.cuda.synchronize()
    _same("block kernel codes", host(q), qo)
    _same("block kernel scales", host(s), so)
    assert not np.any((qo & 0x7F) == 0x7F)    # no NaN code
