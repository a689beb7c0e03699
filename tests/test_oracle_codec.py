"""Pins for the oracle's E4M3 codec against what the pages and the format fix.

* 448 is the largest finite magnitude and E4M3 has 4 exponent + 3 mantissa
  bits (golden fixture ``tests/golden/e4m3_landmarks.txt`` with citations).
* The decoder agrees with torch's float8_e4m3fn widening (a library routine)
  on all 256 codes.
* The encoder agrees with an exhaustive brute-force nearest-value table search
  over all 2^32 fp32 bit patterns (``tests/pins/e4m3_nearest.c``), and with
  torch's float8_e4m3fn narrowing inside the finite range.
"""
import ctypes
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    rows = []
    with open(os.path.join(HERE, "golden", "e4m3_landmarks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, value = line.split()
            rows.append((int(code, 16), float(value)))
    return rows


ALL = np.arange(256, dtype=np.uint8)


def test_golden_max_448():
    dec = oracle.e4m3_decode(ALL)
    for code, value in _golden():
        assert dec[code] == value
    finite = dec[np.isfinite(dec)]
    assert finite.max() == 448.0 and finite.min() == -448.0


def test_three_mantissa_bits_four_exponent_bits():
    dec = oracle.e4m3_decode(ALL[:0x7F]).astype(np.float64)   # non-negative finite
    assert np.all(np.diff(dec) > 0), "codes 0..0x7E must be increasing"
    # normal binades [2^e, 2^(e+1)) hold 8 evenly spaced values (3 mantissa bits)
    binades = 0
    for e in range(-6, 9):
        lo, hi = 2.0 ** e, 2.0 ** (e + 1)
        vals = dec[(dec >= lo) & (dec < hi)]
        expect = 8 if e < 8 else 7       # top binade loses its last value to NaN
        assert vals.size == expect, (e, vals)
        assert np.allclose(np.diff(vals), 2.0 ** (e - 3))
        binades += 1
    assert binades == 15                 # 4 exponent bits: fields 1..15 are normal
    # subnormals: 7 values spaced by 2^-9 below the min normal 2^-6
    sub = dec[(dec > 0) & (dec < 2.0 ** -6)]
    assert sub.size == 7 and np.allclose(sub, np.arange(1, 8) * 2.0 ** -9)
    assert dec.size - 1 == 126           # 126 positive finite values, 253 distinct overall


def test_decode_matches_torch_all_codes():
    dec = oracle.e4m3_decode(ALL)
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(np.isnan(dec), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(dec[ok].view(np.uint32), ref[ok].view(np.uint32))   # incl. -0
    assert set(np.nonzero(np.isnan(dec))[0].tolist()) == {0x7F, 0xFF}


def test_roundtrip_all_codes():
    dec = oracle.e4m3_decode(ALL)
    assert np.array_equal(oracle.e4m3_encode(dec), ALL)


def test_saturation_and_signed_zero():
    enc = oracle.e4m3_encode
    big = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 1e30, np.inf], np.float32)
    assert np.all(enc(big) == 0x7E)
    assert np.all(enc(-big) == 0xFE)
    assert enc(np.float32(-0.0)) == 0x80 and enc(np.float32(0.0)) == 0x00
    assert enc(np.float32(-1e-30)) == 0x80
    # 2^-10 is halfway between 0 and the smallest subnormal: ties to even -> 0
    assert enc(np.float32(2.0 ** -10)) == 0x00
    assert enc(np.float32(3 * 2.0 ** -10)) == 0x02        # 1.5 units -> 2 (even)
    assert enc(np.float32(np.nextafter(np.float32(2.0 ** -10), np.float32(1)))) == 0x01
    # halfway between 1.0 (0x38) and 1.125 (0x39) -> even mantissa 0x38
    assert enc(np.float32(1.0625)) == 0x38
    assert enc(np.float32(1.1875)) == 0x3A                 # between 0x39 and 0x3A -> 0x3A


def test_encode_matches_torch_in_range():
    g = np.random.Generator(np.random.PCG64(7))
    bits = g.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    bf16_all = (np.arange(1 << 16, dtype=np.uint32) << 16)
    v = np.concatenate([bits, bf16_all]).view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    ref = torch.from_numpy(v.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(v), ref)


@pytest.fixture(scope="module")
def nearest_lib(tmp_path_factory):
    d = tmp_path_factory.mktemp("pins")
    so = str(d / "libnearest.so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC",
                           os.path.join(HERE, "pins", "e4m3_nearest.c"), "-o", so, "-lm"])
    L = ctypes.CDLL(so)
    L.count_mismatches.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32)]
    L.count_mismatches.restype = ctypes.c_int64
    L.nearest_code.argtypes = [ctypes.c_float]
    L.nearest_code.restype = ctypes.c_uint8
    return L


def test_bruteforce_helper_sanity(nearest_lib):
    # the helper itself against hand-checked values
    assert nearest_lib.nearest_code(1.0) == 0x38
    assert nearest_lib.nearest_code(448.0) == 0x7E
    assert nearest_lib.nearest_code(-500.0) == 0xFE
    assert nearest_lib.nearest_code(1.0625) == 0x38
    assert nearest_lib.nearest_code(2.0 ** -9) == 0x01


def test_encode_exhaustive_vs_bruteforce(nearest_lib):
    enc_ptr = ctypes.cast(oracle.lib().orc_e4m3_encode, ctypes.c_void_p)
    first = ctypes.c_uint32()
    bad = nearest_lib.count_mismatches(enc_ptr, ctypes.byref(first))
    assert bad == 0, "first mismatching fp32 pattern 0x%08x" % first.value
