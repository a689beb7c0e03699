"""The FP8 linear step (quantizers, forward, dgrad and wgrad GEMMs) captured
once as a HIP graph and replayed: every replay must reproduce the eagerly
launched step bit for bit.  The library launches only its own kernels on the
caller's stream (no allocation, memset or synchronization), so the whole
step can be captured; the replays are separated by the program's own eager
work (clearing every output) and synchronizations, and each is checked.

Shapes span several GEMM tiles with a ragged edge in every dimension
(M = 640, N = 896, K = 704).
"""
import numpy as np
import pytest
import torch

import fp8_precision_quant_amd as fq
import synthetic
from gpu_util import DEV, host, to_dev_bf16

pytestmark = pytest.mark.gpu

M, N, K = 640, 896, 704


def _step_buffers():
    x = to_dev_bf16(synthetic.normal_bf16((M, K), 901))
    w = to_dev_bf16(synthetic.normal_bf16((N, K), 902, 0.02))
    dy = to_dev_bf16(synthetic.bf16_from_f32(
        synthetic.heavy_tail_f32(synthetic.normal_f32((M, N), 903, 1e-3), 0.001, 904)))
    cd = lambda n: -(-n // 128)
    z = lambda r, c, dt: torch.zeros((r, c), dtype=dt, device=DEV)
    u8, f32 = torch.uint8, torch.float32
    out = dict(
        qx=z(M, K, u8), sx=z(M, cd(K), f32), qw=z(N, K, u8), sw=z(cd(N), cd(K), f32),
        y=z(M, N, torch.bfloat16), qdy=z(M, N, u8), sdy=z(M, cd(N), f32),
        qdyT=z(N, M, u8), sdyT=z(N, cd(M), f32), qxT=z(K, M, u8), sxT=z(K, cd(M), f32),
        dx=z(M, K, torch.bfloat16), dW=z(N, K, f32))
    return x, w, dy, out


def _step(x, w, dy, o):
    fq.fp8_quant_blockwise(x, fq.ROW_1x128, q=o["qx"], s=o["sx"])
    fq.fp8_quant_blockwise(w, fq.BLOCK_128x128, q=o["qw"], s=o["sw"])
    fq.fp8_gemm_blockscaled(o["qx"], o["sx"], fq.ROW_1x128, o["qw"], o["sw"], fq.BLOCK_128x128,
                            fq.B_NK, c=o["y"])
    fq.fp8_quant_transpose(dy, out=(o["qdy"], o["sdy"], o["qdyT"], o["sdyT"]))
    fq.fp8_quant_transpose(x, rows_out=False, out=(None, None, o["qxT"], o["sxT"]))
    fq.fp8_gemm_blockscaled(o["qdy"], o["sdy"], fq.ROW_1x128, o["qw"], o["sw"], fq.BLOCK_128x128,
                            fq.B_KN, c=o["dx"])
    fq.fp8_gemm_blockscaled(o["qdyT"], o["sdyT"], fq.ROW_1x128, o["qxT"], o["sxT"], fq.ROW_1x128,
                            fq.B_NK, c=o["dW"])


def test_step_graph_replays_match_eager():
    x, w, dy, o = _step_buffers()
    _step(x, w, dy, o)
    torch.cuda.synchronize()
    eager = {k: host(v).copy() for k, v in o.items()}
    for k, v in eager.items():
        assert np.any(v != 0), "eager step left %s empty" % k

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(x, w, dy, o)
    for rep in range(3):
        for v in o.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in o.items():
            assert np.array_equal(host(v), eager[k]), "replay %d differs from eager in %s" % (rep, k)
