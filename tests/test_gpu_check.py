"""The debug mode FP8Q_CHECK=1 on the device: before a grouped GEMM is
enqueued, a check kernel validates the group-offset contract (off[0] = 0,
non-decreasing, every offset a multiple of 128, off[G] <= M_pad; the padded
routing map of the Ling 2.0 FP8 blog, "FP8 padding routing map").  A
violation returns FP8Q_ERR_SHAPE and enqueues no GEMM (the output keeps its
sentinel); valid offsets give the same bytes as without the check.  The
forward is checked with both outputs (fp32, and E4M3 codes with scales).

Every violating offset vector used here stays within [0, M_pad], and those
given to the backward kernels are also non-decreasing, so the GEMM would
still stay inside its buffers if the check let one through.  A violation the
kernels could not survive (off[G] > M_pad) is never run on the device.
"""
import numpy as np
import pytest
import torch

import fp8_precision_quant_amd as fq
from gpu_util import DEV, host, to_dev

pytestmark = pytest.mark.gpu

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
G, M_PAD, N, K = 3, 384, 256, 256


def _codes(shape, seed):
    return to_dev(np.random.Generator(np.random.PCG64(seed)).choice(FINITE, size=shape))


def _scales(shape, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return to_dev((np.exp(g.standard_normal(shape)) * 0.01).astype(np.float32))


@pytest.fixture(scope="module")
def operands():
    return dict(a=_codes((M_PAD, K), 1), sa=_scales((M_PAD, K // 128), 2), b=_codes((G, N, K), 3),
                sb=_scales((G, N // 128, K // 128), 4),
                dy=_codes((M_PAD, N), 5), sdy=_scales((M_PAD, N // 128), 6),
                at=_codes((N, M_PAD), 7), sat=_scales((N, M_PAD // 128), 8),
                bt=_codes((K, M_PAD), 9), sbt=_scales((K, M_PAD // 128), 10))


def _off(values):
    return torch.tensor(values, dtype=torch.int32, device=DEV)


def _fwd(o, off, c):
    return fq.fp8_grouped_gemm(o["a"], o["sa"], off, o["b"], o["sb"], out_dtype=torch.float32, c=c)


def _fwd_e4m3(o, off, c):
    q, sc = c
    return fq.fp8_grouped_gemm_e4m3(o["a"], o["sa"], off, o["b"], o["sb"], q=q, s=sc)


def _dgrad(o, off, c):
    return fq.fp8_grouped_gemm_dgrad(o["dy"], o["sdy"], off, o["b"], o["sb"], out_dtype=torch.float32, c=c)


def _wgrad(o, off, c):
    return fq.fp8_grouped_gemm_wgrad(o["at"], o["sat"], o["bt"], o["sbt"], off, c=c)


def _out(kind):
    if kind == "fwd_e4m3":
        return (torch.full((M_PAD, N), 0x5A, dtype=torch.uint8, device=DEV),
                torch.full((M_PAD, N // 128), -7.0, dtype=torch.float32, device=DEV))
    shape = {"fwd": (M_PAD, N), "dgrad": (M_PAD, K), "wgrad": (G, N, K)}[kind]
    return torch.full(shape, -7.0, dtype=torch.float32, device=DEV)


def _bytes(c):
    parts = c if isinstance(c, tuple) else (c,)
    return b"".join(host(t).tobytes() for t in parts)


def _untouched(c):
    if isinstance(c, tuple):
        return bool((c[0] == 0x5A).all()) and bool((c[1] == -7.0).all())
    return bool((c == -7.0).all())


RUN = {"fwd": _fwd, "fwd_e4m3": _fwd_e4m3, "dgrad": _dgrad, "wgrad": _wgrad}


@pytest.mark.parametrize("kind", ["fwd", "fwd_e4m3", "dgrad", "wgrad"])
def test_valid_offsets_run_unchanged(operands, kind, monkeypatch):
    off = _off([0, 128, 128, 384])                  # an empty middle group
    monkeypatch.delenv("FP8Q_CHECK", raising=False)
    plain = _out(kind)
    RUN[kind](operands, off, plain)
    torch.cuda.synchronize()
    monkeypatch.setenv("FP8Q_CHECK", "1")
    checked = _out(kind)
    RUN[kind](operands, off, checked)
    torch.cuda.synchronize()
    assert _bytes(plain) == _bytes(checked)


@pytest.mark.parametrize("values, what", [
    ([0, 100, 256, 384], "offset not a multiple of 128"),
    ([0, 256, 128, 384], "decreasing offsets"),
    ([128, 256, 256, 384], "first offset not zero"),
])
@pytest.mark.parametrize("kind", ["fwd", "fwd_e4m3"])
def test_forward_violations_are_reported(operands, kind, values, what, monkeypatch):
    monkeypatch.setenv("FP8Q_CHECK", "1")
    c = _out(kind)
    with pytest.raises(fq.Fp8qError) as err:
        RUN[kind](operands, _off(values), c)
    assert err.value.status == fq.ERR_SHAPE, what
    torch.cuda.synchronize()
    assert _untouched(c), "the GEMM ran despite " + what


@pytest.mark.parametrize("kind", ["dgrad", "wgrad"])
def test_backward_violation_is_reported(operands, kind, monkeypatch):
    monkeypatch.setenv("FP8Q_CHECK", "1")
    c = _out(kind)
    with pytest.raises(fq.Fp8qError) as err:
        RUN[kind](operands, _off([0, 100, 256, 384]), c)
    assert err.value.status == fq.ERR_SHAPE
    torch.cuda.synchronize()
    assert _untouched(c)
