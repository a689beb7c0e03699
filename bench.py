#!/usr/bin/env python3
"""Benchmark of the FP8 linear-layer hot path on one MI355X.

One step = one training pass of an FP8 Linear with block-scaled E4M3
operands on the MLP up-projection shape (x [4096 x 4096] bf16 ~N(0,1),
W [14336 x 4096] bf16 ~N(0,0.02), dy [4096 x 14336] bf16 ~1e-3 N(0,1) with
0.1% heavy-tailed outliers):

  forward   x       -> quant + transpose (rows and columns; one read of x,
                       the transposed codes are kept for the backward)
            qW,sW   = quant 128x128 (W)          y  = gemm(qx, qW^T)   bf16 out
  backward  dy      -> quant + transpose (rows and columns)
            dx = gemm(q_row(dy), qW stored [N][K] read as KN)          bf16 out
            dW = gemm(q_colT(dy), q_colT(x), row x row scales)          fp32 out

All inputs are resident in HBM before the timed region.  `value` is the
GEMM work of the step (3 x 2*M*N*K) divided by the GPU time of the whole
step, quantizers included (K steps between two events, nothing else in
between).  A second pass over K steps brackets each launch with events for
the per-kernel breakdown.  The roofline entry covers the kernel that takes
the most time in the step; the per-kernel breakdown is reported alongside.
The CPU baseline times the oracle on a bounded sample of the same step.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-scaled FP8 GEMM TFLOPS (% FP8 MFMA peak); quantizer GB/s (% HBM)"
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E

M, N, K = 4096, 14336, 4096     # tokens, out features (14336), in features

# HBM traffic per launch comes from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
# scaled by the same counters on a plain copy of known size, and is recorded
# with a hash of the kernel's sources; a changed kernel reports null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_mlp_fwd_bwd_step.txt")
CSRC = os.path.join(ROOT, "fp8_precision_quant_amd", "csrc")
KERNEL_SOURCES = {
    "quant": ["quant.hip", "fp8q_device.h"],
    "quant_transpose": ["quant_transpose.hip", "fp8q_device.h"],
    "gemm": ["gemm_nk.hip", "gemm.hip", "gemm_common.h", "fp8q_device.h"],
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-moe", action="store_true", help="skip the grouped MoE GEMM timing")
    p.add_argument("--cpu-rows", type=int, default=4096,
                   help="output rows per GEMM in the oracle's timed sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device-to-device copy (5 times), the reference "
                        "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters")
    return p.parse_args()


def source_hash(group):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[group]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(op_name, group):
    """HBM bytes per launch of `op_name` from the recorded counter summary,
    or None if absent or taken on different kernel sources."""
    import configparser
    if not os.path.exists(TRAFFIC_FILE):
        return None
    cp = configparser.ConfigParser(comment_prefixes=("#",), interpolation=None)
    cp.read(TRAFFIC_FILE)
    if op_name not in cp or cp[op_name].get("source_sha256") != source_hash(group):
        return None
    return int(cp[op_name]["hbm_bytes_per_launch"])


def copy_calibration():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 5}))


def copy_ceiling_gbs(dev):
    """Read+write bandwidth of a plain 1 GiB device-to-device copy (larger
    than the 256 MB last-level cache): the practical HBM ceiling for a
    stream that reads and writes, reported next to the nominal 8 TB/s."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 5
    del src, dst
    return round(2 * n / (ms * 1e-3) / 1e9, 1)


def moe_grouped(dev, reps=10):
    """Grouped MoE GEMMs (outside the step): 8192 tokens, hidden 2048, 128
    experts of intermediate 768, top-8 seeded Zipf(1.1) routing, groups padded
    to 128 rows; random operands generated on the device.  For each expert
    layer: the forward, and the backward's dgrad (expert weight read as
    stored) and wgrad (per-expert token ranges, transposed re-quantized
    operands, fp32 out).  TFLOP/s count the real (unpadded) rows only."""
    import torch
    import fp8_precision_quant_amd as fq
    import synthetic

    T, H, G, I, topk = 8192, 2048, 128, 768, 8
    choice = synthetic.zipf_topk_routing(T, G, topk, 1.1, 402)
    counts = np.bincount(choice.reshape(-1), minlength=G).astype(np.int64)
    padded = -(-counts // 128) * 128
    offsets = np.zeros(G + 1, np.int64)
    offsets[1:] = np.cumsum(padded)
    M_pad = int(offsets[-1])
    off = torch.from_numpy(offsets.astype(np.int32)).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    st = torch.cuda.current_stream(dev)

    def timed(fn):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(st)
        for _ in range(reps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    out = {"tokens": T, "experts": G, "topk": topk, "real_rows": int(counts.sum()), "M_pad": M_pad}
    for name, N, K in (("gate_up", 2 * I, H), ("down", H, I)):
        a = torch.randn((M_pad, K), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        dy = (1e-3 * torch.randn((M_pad, N), generator=gen, device=dev, dtype=torch.float32)).to(torch.bfloat16)
        w = (0.02 * torch.randn((G * N, K), generator=gen, device=dev, dtype=torch.float32)).to(torch.bfloat16)
        qa, sa = fq.fp8_quant_blockwise(a, fq.ROW_1x128)
        qw, sw = fq.fp8_quant_blockwise(w, fq.BLOCK_128x128)
        qw = qw.view(G, N, K)
        sw = sw.view(G, -(-N // 128), -(-K // 128))
        qdy, sdy, qdyT, sdyT = fq.fp8_quant_transpose(dy)
        _, _, qaT, saT = fq.fp8_quant_transpose(a, rows_out=False)
        c = torch.empty((M_pad, N), dtype=torch.bfloat16, device=dev)
        dx = torch.empty((M_pad, K), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((G, N, K), dtype=torch.float32, device=dev)
        flops = 2.0 * counts.sum() * N * K
        res = {"N": N, "K": K}
        for part, fn in (("fwd", lambda: fq.fp8_grouped_gemm(qa, sa, off, qw, sw, c=c)),
                         ("dgrad", lambda: fq.fp8_grouped_gemm_dgrad(qdy, sdy, off, qw, sw, c=dx)),
                         ("wgrad", lambda: fq.fp8_grouped_gemm_wgrad(qdyT, sdyT, qaT, saT, off, c=dw))):
            us = timed(fn)
            res[part] = {"us": round(us, 2), "TFLOP/s": round(flops / (us * 1e-6) / 1e12, 1),
                         "frac_peak": round(flops / (us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4)}
        out[name] = res
        del a, dy, w, qa, sa, qw, sw, qdy, sdy, qdyT, sdyT, qaT, saT, c, dx, dw
    return out


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py: this build measures one GPU; --gpus %d is not supported "
              "(the design notes describe how the path would shard)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_precision_quant_amd as fq
    import synthetic

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x_bits, w_bits = synthetic.mlp_forward(M, N, K)
    dy_bits = synthetic.mlp_backward_dy(M, N)
    x, w, dy = bf16_dev(x_bits), bf16_dev(w_bits), bf16_dev(dy_bits)

    u8, f32 = torch.uint8, torch.float32
    KB, NB, MB = K // 128, N // 128, M // 128
    qx, sx = torch.empty((M, K), dtype=u8, device=dev), torch.empty((M, KB), dtype=f32, device=dev)
    qw, sw = torch.empty((N, K), dtype=u8, device=dev), torch.empty((NB, KB), dtype=f32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    qdy, sdy = torch.empty((M, N), dtype=u8, device=dev), torch.empty((M, NB), dtype=f32, device=dev)
    qdyT, sdyT = torch.empty((N, M), dtype=u8, device=dev), torch.empty((N, MB), dtype=f32, device=dev)
    qxT, sxT = torch.empty((K, M), dtype=u8, device=dev), torch.empty((K, MB), dtype=f32, device=dev)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((N, K), dtype=f32, device=dev)

    gemm_flops = 2.0 * M * N * K
    # algorithmic bytes: what each kernel must read and write at least
    ops = [
        ("quant_transpose x", lambda: fq.fp8_quant_transpose(x, out=(qx, sx, qxT, sxT)),
         "hbm", M * K * 2 + 2 * M * K + 4 * (M * KB + K * MB)),
        ("quant_128x128 W", lambda: fq.fp8_quant_blockwise(w, fq.BLOCK_128x128, q=qw, s=sw),
         "hbm", N * K * 2 + N * K + NB * KB * 4),
        ("gemm fwd y=xW^T", lambda: fq.fp8_gemm_blockscaled(qx, sx, fq.ROW_1x128, qw, sw,
                                                           fq.BLOCK_128x128, fq.B_NK, c=y),
         "mfma", gemm_flops),
        ("quant_transpose dy", lambda: fq.fp8_quant_transpose(dy, out=(qdy, sdy, qdyT, sdyT)),
         "hbm", M * N * 2 + 2 * M * N + 4 * (M * NB + N * MB)),
        ("gemm dgrad dx=dyW", lambda: fq.fp8_gemm_blockscaled(qdy, sdy, fq.ROW_1x128, qw, sw,
                                                             fq.BLOCK_128x128, fq.B_KN, c=dx),
         "mfma", gemm_flops),
        ("gemm wgrad dW=dy^T x", lambda: fq.fp8_gemm_blockscaled(qdyT, sdyT, fq.ROW_1x128, qxT, sxT,
                                                                fq.ROW_1x128, fq.B_NK, c=dW),
         "mfma", gemm_flops),
    ]

    group_of = {"quant_transpose x": "quant_transpose", "quant_128x128 W": "quant",
                "quant_transpose dy": "quant_transpose"}

    def step():
        for _, fn, _, _ in ops:
            fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region 1: the whole step, K times, bracketed by synchronizations;
    # no events inside the step
    stream = torch.cuda.current_stream(dev)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps


    # timed region 2: the same K steps with an event pair around every launch
    # (on the launch stream) for per-kernel durations; events add a few us to
    # each launch, which matters only for the short quantizer kernels
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, (_, fn, _, _) in enumerate(ops):
            fn()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()

    per_op_ms = np.zeros(len(ops))
    for s in range(args.steps):
        for i in range(len(ops)):
            per_op_ms[i] += ev[s][i].elapsed_time(ev[s][i + 1])
    per_op_ms /= args.steps

    step_flops = 3 * gemm_flops
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    breakdown = []
    for (name, _, bound, work), t in zip(ops, per_op_ms):
        if bound == "mfma":
            ach = work / (t * 1e-3) / 1e12
            breakdown.append({"kernel": name, "us": round(t * 1e3, 2), "TFLOP/s": round(ach, 1),
                              "frac_peak": round(ach / PEAK_FP8_TFLOPS, 4)})
        else:
            ach = work / (t * 1e-3) / 1e9
            breakdown.append({"kernel": name, "us": round(t * 1e3, 2), "GB/s": round(ach, 1),
                              "frac_peak": round(ach / PEAK_HBM_GBS, 4)})
    dom = int(np.argmax(per_op_ms))
    dname, _, dbound, dwork = ops[dom]
    dt = per_op_ms[dom] * 1e-3
    traffic = recorded_traffic(dname, group_of.get(dname, "gemm"))
    if dbound == "mfma":
        roofline = {"bound": "mfma", "achieved": round(dwork / dt / 1e12, 2), "peak": PEAK_FP8_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(dwork / dt / 1e12 / PEAK_FP8_TFLOPS, 4),
                    "traffic": traffic, "kernel": dname}
    else:
        roofline = {"bound": "hbm", "achieved": round(dwork / dt / 1e9, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(dwork / dt / 1e9 / PEAK_HBM_GBS, 4),
                    "traffic": traffic, "kernel": dname}
    roofline["traffic_unit"] = "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    hbm_copy = copy_ceiling_gbs(dev)
    moe = None if args.no_moe else moe_grouped(dev)

    # The forward GEMM storing its output quantized (E4M3 codes + 1x128
    # scales: the next layer's activation quantization) against the same GEMM
    # with bf16 output followed by the separate 1x128 quantization of y.
    qy = torch.empty((M, N), dtype=u8, device=dev)
    sy = torch.empty((M, NB), dtype=f32, device=dev)
    fused = {}
    for name, fn in (
            ("gemm_bf16_out", lambda: fq.fp8_gemm_blockscaled(qx, sx, fq.ROW_1x128, qw, sw, fq.BLOCK_128x128,
                                                              fq.B_NK, c=y)),
            ("quant_1x128_y", lambda: fq.fp8_quant_blockwise(y, fq.ROW_1x128, q=qy, s=sy)),
            ("gemm_e4m3_out", lambda: fq.fp8_gemm_blockscaled_e4m3(qx, sx, fq.ROW_1x128, qw, sw, fq.BLOCK_128x128,
                                                                   fq.B_NK, out=(qy, sy)))):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        fused[name + "_us"] = round(e0.elapsed_time(e1) * 1e3 / args.steps, 2)
    fused["saving_us"] = round(fused["gemm_bf16_out_us"] + fused["quant_1x128_y_us"] - fused["gemm_e4m3_out_us"], 2)

    # The same step with power-of-two scales (E8M0 bytes; the scaled MFMA
    # applies them): per-launch times of each kernel.
    def e8(rows, cols):
        return torch.empty((rows, (cols + 3) // 4 * 4), dtype=u8, device=dev)[:, :cols]
    ex, ew, edy, edyT, exT = e8(M, KB), e8(NB, KB), e8(M, NB), e8(N, MB), e8(K, MB)
    p2_ops = [
        ("quant_transpose x", lambda: fq.fp8_quant_transpose_e8m0(x, out=(qx, ex, qxT, exT)),
         M * K * 2 + 2 * M * K + M * KB + K * MB),
        ("quant_128x128 W", lambda: fq.fp8_quant_blockwise_e8m0(w, fq.BLOCK_128x128, q=qw, e=ew),
         N * K * 2 + N * K + NB * KB),
        ("gemm fwd y=xW^T", lambda: fq.fp8_gemm_e8m0(qx, ex, qw, ew, fq.BLOCK_128x128, fq.B_NK, c=y), None),
        ("quant_transpose dy", lambda: fq.fp8_quant_transpose_e8m0(dy, out=(qdy, edy, qdyT, edyT)),
         M * N * 2 + 2 * M * N + M * NB + N * MB),
        ("gemm dgrad dx=dyW", lambda: fq.fp8_gemm_e8m0(qdy, edy, qw, ew, fq.BLOCK_128x128, fq.B_KN, c=dx), None),
        ("gemm wgrad dW=dy^T x", lambda: fq.fp8_gemm_e8m0(qdyT, edyT, qxT, exT, fq.ROW_1x128, fq.B_NK, c=dW),
         None),
    ]
    # timed like the main step: K whole steps between two events, then K
    # steps with an event pair around every launch
    for _ in range(args.warmup):
        for _, fn, _ in p2_ops:
            fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        for _, fn, _ in p2_ops:
            fn()
    e1.record(stream)
    torch.cuda.synchronize()
    p2_step_ms = e0.elapsed_time(e1) / args.steps
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(len(p2_ops) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for st_i in range(args.steps):
        ev2[st_i][0].record(stream)
        for i, (_, fn, _) in enumerate(p2_ops):
            fn()
            ev2[st_i][i + 1].record(stream)
    torch.cuda.synchronize()
    pow2 = {"ms_per_step": round(p2_step_ms, 4),
            "TFLOP/s": round(step_flops / (p2_step_ms * 1e-3) / 1e12, 2), "kernels": []}
    for i, (name, _, hbm_bytes) in enumerate(p2_ops):
        us = sum(ev2[st_i][i].elapsed_time(ev2[st_i][i + 1]) for st_i in range(args.steps)) * 1e3 / args.steps
        rec = {"kernel": name, "us": round(us, 2)}
        if name.startswith("gemm"):
            rec["TFLOP/s"] = round(gemm_flops / (us * 1e-6) / 1e12, 1)
            rec["frac_peak"] = round(gemm_flops / (us * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4)
        else:
            rec["GB/s"] = round(hbm_bytes / (us * 1e-6) / 1e9, 1)
            rec["frac_peak"] = round(hbm_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        pow2["kernels"].append(rec)

    # The optimizer step of the same layer: AdamW with FP8 moments on an fp32
    # master copy of W, the step's fp32 dW as gradient.
    n_w = N * K
    p_w = w.float().reshape(-1).contiguous()
    g_w = dW.reshape(-1)
    st8 = fq.fp8_adam_state(n_w, dev)
    for t in range(1, args.warmup + 1):
        fq.fp8_adam_step(p_w, g_w, st8, lr=1e-4, weight_decay=0.1, step=t)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(args.warmup + 1, args.warmup + 1 + args.steps):
        fq.fp8_adam_step(p_w, g_w, st8, lr=1e-4, weight_decay=0.1, step=t)
    e1.record(stream)
    torch.cuda.synchronize()
    adam_us = e0.elapsed_time(e1) * 1e3 / args.steps
    # algorithmic bytes: parameters read and written (8), fp32 gradient (4),
    # both moments' codes read and written (4), their scales (16 per 128)
    adam_bytes = n_w * 16 + (n_w // 128) * 16
    adam = {"params": n_w, "us": round(adam_us, 2), "GB/s": round(adam_bytes / (adam_us * 1e-6) / 1e9, 1),
            "frac_peak": round(adam_bytes / (adam_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "state_bytes_per_param": 2 + 8 / 128}
    del p_w, st8

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x_bits, w_bits, dy_bits, args.cpu_rows)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 x fp8-e4m3 -> f32 accumulate",
        "data": "synthetic (seeded numpy; no dataset)",
        "config": {"workload": "FP8 linear fwd+bwd, MLP up-proj x[4096x4096] W[14336x4096] dy[4096x14336], "
                               "1x128 act/grad tiles, 128x128 weight blocks, E4M3",
                   "M": M, "N": N, "K": K, "gemm_flops_per_step": step_flops,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "kernels": breakdown,
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
        "hbm_copy_GBps": hbm_copy,
        "moe_grouped": moe,
        "fwd_quantize_on_store": fused,
        "pow2_scales": pow2,
        "fp8_adam": adam,
    }
    print(json.dumps(out))


def cpu_baseline(x_bits, w_bits, dy_bits, rows_per_gemm):
    """The oracle on a bounded sample of the same step: full-tensor quantizers
    for x (1x128) and W (128x128) and the three GEMMs on `rows_per_gemm`
    output rows each; reported as GEMM TFLOP/s of the sample."""
    import oracle
    import synthetic

    t0 = time.perf_counter()
    xf = synthetic.bf16_to_f32(x_bits)
    wf = synthetic.bf16_to_f32(w_bits)
    t_q0 = time.perf_counter()
    qx, sx = oracle.quant_1x128(xf)
    qw, sw = oracle.quant_128x128(wf)
    t_q = time.perf_counter() - t_q0
    q_bytes = xf.size * 3 + wf.size * 3
    dyf = synthetic.bf16_to_f32(dy_bits)
    t_t0 = time.perf_counter()
    qdy, sdy, qdyT, sdyT = oracle.quant_transpose(dyf)
    _, _, qxT, sxT = oracle.quant_transpose(xf)
    t_t = time.perf_counter() - t_t0
    rows = synthetic.sample_rows(M, rows_per_gemm, 7)
    rows_w = synthetic.sample_rows(N, 2 * rows_per_gemm, 8)
    t_g0 = time.perf_counter()
    oracle.gemm_blockscaled(qx, sx, "row", qw, sw, "block", "NK", rows=rows)
    oracle.gemm_blockscaled(qdy, sdy, "row", qw, sw, "block", "KN", rows=rows)
    oracle.gemm_blockscaled(qdyT, sdyT, "row", qxT, sxT, "row", "NK", rows=rows_w)
    t_g = time.perf_counter() - t_g0
    flops = 2.0 * len(rows) * N * K + 2.0 * len(rows) * K * N + 2.0 * len(rows_w) * K * M
    return {"value": round(flops / t_g / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "quant 1x128 x + 128x128 W (full tensors, %.1f GB/s), quant+transpose of dy and x "
                      "(full, %.2f s), and fwd/dgrad GEMMs on all %d rows, wgrad on %d sampled rows "
                      "(%.2f s); value = GEMM FLOPs of the sample / GEMM time"
                      % (q_bytes / t_q / 1e9, t_t, len(rows), len(rows_w), t_g),
            "total_s": round(time.perf_counter() - t0, 2)}


if __name__ == "__main__":
    main()
