"""GPU parity of the AdamW step with FP8 moments (fp8_adam_step) against the
oracle.

The step is a fixed sequence of fp32 roundings followed by the 1x128 tile
quantization, so the bar is bit-exact: parameter bits, moment codes and
scale bits.  The GPU and the oracle each run their own chain of steps from
the same seeded start (the oracle never sees a GPU result).  Cases: sizes
with ragged last blocks (1, 127, 128, 300, 4097, 1 000 003), fp32 and bf16
gradients, weight decay on and off, late steps (bias correction near 1), a
fresh all-zero state, zero gradients, canaries around every output, and the
MLP weight's size (58.7 M parameters).
"""
import numpy as np
import pytest
import torch

import fp8_precision_quant_amd as fq
import oracle
import synthetic
from gpu_util import DEV, host

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _start(n, seed, fresh=False):
    p, g, m, v = synthetic.adam_inputs(n, seed)
    if fresh:
        z8, zs = np.zeros(n, np.uint8), np.zeros(-(-n // 128), np.float32)
        return p, g, (z8, zs, z8.copy(), zs.copy())
    mq, ms = oracle.quant_1x128(m[None, :])
    vq, vs = oracle.quant_1x128(v[None, :])
    return p, g, (mq[0], ms[0], vq[0], vs[0])


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _compare(step, dp, dstate, op, ostate):
    names = ["p", "mq", "ms", "vq", "vs"]
    got = [host(dp)] + [host(t) for t in dstate]
    want = [op] + list(ostate)
    for name, a, b in zip(names, got, want):
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        bad = np.flatnonzero(a != b)
        assert bad.size == 0, "step %d: %s differs at %s (gpu %s, oracle %s)" % (
            step, name, bad[:5].tolist(), a[bad[0]], b[bad[0]])


def _run_chain(n, seed, g_dtype, wd, steps, first_step=1, fresh=False, zero_grad=False):
    p, g, state = _start(n, seed, fresh)
    if zero_grad:
        g = np.zeros_like(g)
    if g_dtype == "bf16":
        gbits = synthetic.bf16_from_f32(g)
        g = synthetic.bf16_to_f32(gbits)
        dg = _dev(gbits.view(np.int16)).view(torch.bfloat16)
    else:
        dg = _dev(g)
    dp = _dev(p)
    dstate = tuple(_dev(s) for s in state)
    op, ostate = p, state
    for t in range(first_step, first_step + steps):
        fq.fp8_adam_step(dp, dg, dstate, step=t, weight_decay=wd, **HP)
        torch.cuda.synchronize()
        out = oracle.adamw_fp8_step(op, g, *ostate, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], wd, t)
        op, ostate = out[0], out[1:]
        _compare(t, dp, dstate, op, ostate)


@pytest.mark.parametrize("n", [1, 127, 128, 300, 4097, 1000003])
@pytest.mark.parametrize("g_dtype", ["f32", "bf16"])
def test_parity_over_steps(n, g_dtype):
    _run_chain(n, 610 + n % 97, g_dtype, wd=0.1, steps=3)


def test_no_weight_decay_and_late_steps():
    _run_chain(5000, 620, "f32", wd=0.0, steps=2, first_step=1000)


def test_fresh_state():
    _run_chain(3000, 621, "bf16", wd=0.01, steps=3, fresh=True)


def test_zero_gradient():
    _run_chain(1000, 622, "f32", wd=0.1, steps=2, zero_grad=True)


def test_canaries():
    n = 300
    p, g, (mq, ms, vq, vs) = _start(n, 623)
    pb = torch.full((n + 64,), -7.0, dtype=torch.float32, device=DEV)
    mqb = torch.full((n + 64,), 0x5A, dtype=torch.uint8, device=DEV)
    vqb = torch.full((n + 64,), 0x5A, dtype=torch.uint8, device=DEV)
    msb = torch.full((8,), -9.0, dtype=torch.float32, device=DEV)
    vsb = torch.full((8,), -9.0, dtype=torch.float32, device=DEV)
    pb[:n] = _dev(p)
    mqb[:n] = _dev(mq)
    vqb[:n] = _dev(vq)
    msb[:3] = _dev(ms)
    vsb[:3] = _dev(vs)
    fq.fp8_adam_step(pb[:n], _dev(g), (mqb[:n], msb[:3], vqb[:n], vsb[:3]), step=2, weight_decay=0.1, **HP)
    torch.cuda.synchronize()
    assert torch.all(pb[n:].cpu() == -7.0)
    assert torch.all(mqb[n:].cpu() == 0x5A) and torch.all(vqb[n:].cpu() == 0x5A)
    assert torch.all(msb[3:].cpu() == -9.0) and torch.all(vsb[3:].cpu() == -9.0)
    out = oracle.adamw_fp8_step(p, g, mq, ms, vq, vs, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], 0.1, 2)
    _compare(2, pb[:n], (mqb[:n], msb[:3], vqb[:n], vsb[:3]), out[0], out[1:])


def test_mlp_weight_size():
    """One step on the MLP weight's 14336 x 4096 parameters, bit-exact."""
    _run_chain(14336 * 4096, 630, "f32", wd=0.1, steps=1)
