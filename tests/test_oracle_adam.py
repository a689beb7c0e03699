"""Pins of the oracle's Adam step with FP8 moments (Ling 2.0 FP8 blog, "FP8
Optimizer": Adam's first and second moments held in FP8 through fine-grained
compression; it points to block-wise quantization).

The fp32 step is pinned to torch.optim.AdamW (a library routine for the same
textbook algorithm) and to the closed form of the first step; the FP8 step is
pinned as decode -> fp32 step -> 1x128 quantization of the separately pinned
pieces, plus the pages' claim that FP8 moments hardly change convergence.
"""
import numpy as np
import pytest
import torch

import oracle

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.1)


def _torch_adamw(p0, grads, **hp):
    p = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([p], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["wd"], foreach=False, fused=False)
    for g in grads:
        p.grad = torch.from_numpy(g.copy())
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_fp32_step_matches_torch_adamw(wd):
    rng = np.random.default_rng(1)
    n = 1000
    p = rng.standard_normal(n).astype(np.float32)
    grads = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-4, 1, n)).astype(np.float32) for _ in range(6)]
    hp = dict(HP, wd=wd)
    pt, mt, vt = _torch_adamw(p, grads, **hp)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    q = p
    for t, g in enumerate(grads, 1):
        q, m, v = oracle.adamw_step(q, g, m, v, hp["lr"], hp["beta1"], hp["beta2"], hp["eps"], hp["wd"], t)
    # torch forms m with lerp and the decay factor in double: a few ulps apart
    # (absolutely, where b1 m and (1-b1) g nearly cancel)
    np.testing.assert_allclose(m, mt, rtol=1e-5, atol=1e-7 * np.abs(mt).max())
    np.testing.assert_allclose(v, vt, rtol=1e-5, atol=0)
    np.testing.assert_allclose(q, pt, rtol=0, atol=1e-6)
    assert np.abs(q - p).max() > 1e-3            # the parameters did move


def test_first_step_closed_form():
    # from zero moments: m = (1-b1) g, v = (1-b2) g^2, and after bias
    # correction the update is lr * g / (|g| + eps)
    rng = np.random.default_rng(2)
    n = 500
    p = rng.standard_normal(n).astype(np.float32)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 2, n)).astype(np.float32)
    q, m, v = oracle.adamw_step(p, g, np.zeros(n, np.float32), np.zeros(n, np.float32), t=1, **_args(HP))
    np.testing.assert_allclose(m, 0.1 * g.astype(np.float64), rtol=2e-7)
    np.testing.assert_allclose(v, 0.001 * g.astype(np.float64) ** 2, rtol=3e-7)
    g64 = g.astype(np.float64)
    want = p.astype(np.float64) * (1 - 1e-4) - 1e-3 * g64 / (np.abs(g64) + 1e-8)
    np.testing.assert_allclose(q, want, rtol=0, atol=3e-7)


def _args(hp):
    return dict(lr=hp["lr"], beta1=hp["beta1"], beta2=hp["beta2"], eps=hp["eps"], wd=hp["wd"])


@pytest.mark.parametrize("n", [1, 127, 128, 300, 4096])
def test_fp8_step_is_decode_step_quantize(n):
    rng = np.random.default_rng(n)
    p = rng.standard_normal(n).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    nb = -(-n // 128)
    # a state from an earlier step (codes with their scales)
    mq, ms = oracle.quant_1x128((rng.standard_normal(n) * 1e-2).astype(np.float32)[None, :])
    vq, vs = oracle.quant_1x128((rng.random(n) * 1e-4).astype(np.float32)[None, :])
    mq, ms, vq, vs = mq[0], ms[0], vq[0], vs[0]
    assert ms.size == nb
    out = oracle.adamw_fp8_step(p, g, mq, ms, vq, vs, **_args(HP), t=7)
    dec = oracle.e4m3_decode(np.arange(256, dtype=np.uint8))
    m0 = dec[mq] * np.repeat(ms, 128)[:n]
    v0 = dec[vq] * np.repeat(vs, 128)[:n]
    q, m1, v1 = oracle.adamw_step(p, g, m0, v0, **_args(HP), t=7)
    qm, sm = oracle.quant_1x128(m1[None, :])
    qv, sv = oracle.quant_1x128(v1[None, :])
    assert np.array_equal(out[0].view(np.uint32), q.view(np.uint32))
    assert np.array_equal(out[1], qm[0]) and np.array_equal(out[2].view(np.uint32), sm[0].view(np.uint32))
    assert np.array_equal(out[3], qv[0]) and np.array_equal(out[4].view(np.uint32), sv[0].view(np.uint32))


def test_zero_gradient_and_zero_state():
    n = 260
    p = np.linspace(-1, 1, n, dtype=np.float32)
    z8, zs = np.zeros(n, np.uint8), np.zeros(3, np.float32)
    q, mq, ms, vq, vs = oracle.adamw_fp8_step(p, np.zeros(n, np.float32), z8, zs, z8, zs, **_args(HP), t=1)
    np.testing.assert_array_equal(q, p * np.float32(1 - 1e-4))       # decay only: m = 0 gives no update
    assert not mq.any() and not vq.any() and not ms.any() and not vs.any()


def test_fp8_moments_track_fp32_adam_on_least_squares():
    """The pages' claim: FP8 moments, finely scaled, barely change training.
    A least-squares fit (512 parameters, 300 AdamW steps): the FP8-moment run
    reaches a loss within 5% of the fp32 run, along nearly the same path."""
    rng = np.random.default_rng(3)
    A = rng.standard_normal((1024, 512)).astype(np.float32)
    x_true = (rng.standard_normal(512) * 10.0 ** rng.uniform(-2, 0, 512)).astype(np.float32)
    b = A @ x_true + 0.01 * rng.standard_normal(1024).astype(np.float32)

    def grad(x):
        return (A.T @ (A @ x - b) / len(b)).astype(np.float32)

    def loss(x):
        r = A @ x - b
        return float(r @ r) / len(b)

    hp = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0)
    x32 = np.zeros(512, np.float32)
    m = np.zeros(512, np.float32)
    v = np.zeros(512, np.float32)
    x8 = x32.copy()
    mq, ms = np.zeros(512, np.uint8), np.zeros(4, np.float32)
    vq, vs = mq.copy(), ms.copy()
    for t in range(1, 301):
        x32, m, v = oracle.adamw_step(x32, grad(x32), m, v, **hp, t=t)
        x8, mq, ms, vq, vs = oracle.adamw_fp8_step(x8, grad(x8), mq, ms, vq, vs, **hp, t=t)
    l0, l32, l8 = loss(np.zeros(512, np.float32)), loss(x32), loss(x8)
    assert l32 < 1e-2 * l0
    assert l8 <= 1.05 * l32 + 1e-4
    cos = float(x8 @ x32) / (np.linalg.norm(x8) * np.linalg.norm(x32))
    assert cos > 0.99
