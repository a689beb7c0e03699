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

All inputs are resident in HBM before the timed region; consecutive steps
alternate between two complete sets of inputs and outputs, so a step never
finds the previous step's data in the last-level cache.  `value` is the GEMM
work of the step (3 x 2*M*N*K) divided by the GPU time of the whole step,
quantizers included (K steps between two events, nothing else in between).
A second pass over K steps brackets each launch with events for the
per-kernel breakdown.  Timing starts after W warmup steps (default 50, about
50 ms): after an idle gap the clock first drops under the sudden dense load
and recovers over some tens of milliseconds, so a few warmup steps would
time that transient rather than the steady state.  The roofline entry covers the kernel that takes the
most time in the step.

Also reported, each on its own workload (none is part of `value`):
  long_k   x [16384 x 8192] (log-normal rows) and W [8192 x 8192]: 1x128 /
           128x128 / per-tensor quantizers, the blockwise and per-tensor
           GEMMs (bf16 out), underflow fractions, and the error of each
           against the exact product on 256 sampled rows (Frobenius and
           mean per-row), with power-of-two scales alongside;
  moe      8192 tokens, 128 experts, top-8 Zipf routing (the seeded inputs of
           the parity tests): the six grouped launches, with the fraction of
           their attainable roofline max(t_MFMA, t_HBM);
  the quantize-on-store forward, the power-of-two step, the FP8-moment
  AdamW step, the shader clock over a sustained run, and a CPU baseline
  (the oracle on a bounded sample, all host threads and one).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-scaled FP8 GEMM TFLOPS (% FP8 MFMA peak); quantizer GB/s (% HBM)"
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
PEAK_CLOCK_MHZ = 2400.0         # the clock the published FP8 peak assumes

M, N, K = 4096, 14336, 4096     # tokens, out features (14336), in features

# HBM traffic per launch comes from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
# scaled by the same counters on a plain copy of known size, and is recorded
# with a hash of the kernel's sources; a changed kernel reports null.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_mlp_fwd_bwd_step.txt")
CSRC = os.path.join(ROOT, "fp8_precision_quant_amd", "csrc")
KERNEL_SOURCES = {
    "quant": ["quant.hip", "quant_io.h", "fp8q_device.h"],
    "quant_transpose": ["quant_transpose.hip", "quant_io.h", "fp8q_device.h"],
    "gemm": ["gemm_nk.hip", "gemm_w4.hip", "gemm_lds.h", "gemm.hip", "gemm_common.h", "fp8q_device.h"],
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-moe", action="store_true", help="skip the grouped MoE GEMM timing")
    p.add_argument("--no-extras", action="store_true",
                   help="only the step (for profiling): no long-K, MoE, pow2, Adam, clock")
    p.add_argument("--only", default="",
                   help="comma list of parts to run after the step: long_k,moe,e4m3,pow2,adam,clock")
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


def settle(fn_list, ms=60.0):
    """Runs the calls back to back for about `ms` of wall time before a timed
    region.  After an idle gap the first few milliseconds of dense work run
    at a clock the power management then lowers and raises again over tens
    of milliseconds; timing starts past that transient."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn_list[i % len(fn_list)]()
            i += 1
        torch.cuda.synchronize()


def time_launches(fn_list, reps, stream):
    """Average GPU time (us) of one call of each fn: `reps` calls between an
    event pair, fn_list[i % len] in turn (rotating buffer sets), after
    `settle`."""
    import torch
    settle(fn_list)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        fn_list[i % len(fn_list)]()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def gemm_rec(flops, us):
    t = flops / (us * 1e-6) / 1e12
    return {"us": round(us, 2), "TFLOP/s": round(t, 1), "frac_peak": round(t / PEAK_FP8_TFLOPS, 4)}


def hbm_rec(nbytes, us):
    g = nbytes / (us * 1e-6) / 1e9
    return {"us": round(us, 2), "GB/s": round(g, 1), "frac_peak": round(g / PEAK_HBM_GBS, 4)}


def underflow(x, q):
    """Fraction of non-zero inputs whose code has magnitude zero (0x00, 0x80);
    x and q of the same shape, on the device."""
    import torch
    nz = x != 0
    zero_code = (q & 0x7F) == 0
    n = int(nz.sum())
    return float((nz & zero_code).sum()) / n if n else 0.0


def sustained_clock_mhz(dev, fn, seconds=2.5, settle=1.2):
    """Shader clock while `fn` runs back to back for `seconds`, from the
    driver's metrics table (amdsmi gpu_metrics `current_gfxclks`, one clock
    per XCD), sampled every 50 ms.  The table refreshes about once a second
    and its first refresh in the run still averages over the idle time
    before it, so samples of the first `settle` seconds are dropped.  Each
    sample is the mean over the XCDs.  None where the query is unavailable."""
    import torch
    try:
        import amdsmi
        handle = torch.cuda._get_amdsmi_handler(dev)
        amdsmi.amdsmi_get_gpu_metrics_info(handle)
    except Exception:
        return None

    def read():
        clks = amdsmi.amdsmi_get_gpu_metrics_info(handle).get("current_gfxclks")
        clks = [float(c) for c in (clks or []) if isinstance(c, (int, float)) and 0 < c < 65535]
        return clks

    samples = []
    stop = threading.Event()
    t0 = time.perf_counter()

    def sample():
        while not stop.is_set():
            t = time.perf_counter() - t0
            try:
                clks = read()
            except Exception:
                return
            if t >= settle and clks:
                samples.append(clks)
            time.sleep(0.05)

    th = threading.Thread(target=sample)
    th.start()
    while time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None
    means = [float(np.mean(c)) for c in samples]
    per_xcd = np.mean(np.array([c for c in samples if len(c) == len(samples[0])]), axis=0)
    return {"median_mhz": round(float(np.median(means)), 1), "min_mhz": round(min(means), 1),
            "max_mhz": round(max(means), 1), "per_xcd_mhz": [round(float(v)) for v in per_xcd],
            "samples": len(samples), "run_s": seconds,
            "source": "amdsmi gpu_metrics current_gfxclks (mean over XCDs), first %.1f s dropped" % settle}


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
    stream = torch.cuda.current_stream(dev)
    parts = set(p for p in args.only.split(",") if p) or {"long_k", "moe", "e4m3", "pow2", "adam", "clock"}
    if args.no_extras:
        parts = set()
    if args.no_moe:
        parts.discard("moe")

    def bf16_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    x_bits, w_bits = synthetic.mlp_forward(M, N, K)
    dy_bits = synthetic.mlp_backward_dy(M, N)

    u8, f32 = torch.uint8, torch.float32
    KB, NB, MB = K // 128, N // 128, M // 128

    class StepBuffers:
        def __init__(self):
            self.x, self.w, self.dy = bf16_dev(x_bits), bf16_dev(w_bits), bf16_dev(dy_bits)
            self.qx, self.sx = torch.empty((M, K), dtype=u8, device=dev), torch.empty((M, KB), dtype=f32, device=dev)
            self.qw, self.sw = torch.empty((N, K), dtype=u8, device=dev), torch.empty((NB, KB), dtype=f32, device=dev)
            self.y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            self.qdy, self.sdy = torch.empty((M, N), dtype=u8, device=dev), torch.empty((M, NB), dtype=f32, device=dev)
            self.qdyT, self.sdyT = torch.empty((N, M), dtype=u8, device=dev), torch.empty((N, MB), dtype=f32, device=dev)
            self.qxT, self.sxT = torch.empty((K, M), dtype=u8, device=dev), torch.empty((K, MB), dtype=f32, device=dev)
            self.dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
            self.dW = torch.empty((N, K), dtype=f32, device=dev)

    sets = [StepBuffers(), StepBuffers()]

    gemm_flops = 2.0 * M * N * K
    # (name, launch(buffers), bound, algorithmic bytes or FLOPs per launch)
    ops = [
        ("quant_transpose x", lambda b: fq.fp8_quant_transpose(b.x, out=(b.qx, b.sx, b.qxT, b.sxT)),
         "hbm", M * K * 2 + 2 * M * K + 4 * (M * KB + K * MB)),
        ("quant_128x128 W", lambda b: fq.fp8_quant_blockwise(b.w, fq.BLOCK_128x128, q=b.qw, s=b.sw),
         "hbm", N * K * 2 + N * K + NB * KB * 4),
        ("gemm fwd y=xW^T", lambda b: fq.fp8_gemm_blockscaled(b.qx, b.sx, fq.ROW_1x128, b.qw, b.sw,
                                                             fq.BLOCK_128x128, fq.B_NK, c=b.y),
         "mfma", gemm_flops),
        ("quant_transpose dy", lambda b: fq.fp8_quant_transpose(b.dy, out=(b.qdy, b.sdy, b.qdyT, b.sdyT)),
         "hbm", M * N * 2 + 2 * M * N + 4 * (M * NB + N * MB)),
        ("gemm dgrad dx=dyW", lambda b: fq.fp8_gemm_blockscaled(b.qdy, b.sdy, fq.ROW_1x128, b.qw, b.sw,
                                                               fq.BLOCK_128x128, fq.B_KN, c=b.dx),
         "mfma", gemm_flops),
        ("gemm wgrad dW=dy^T x", lambda b: fq.fp8_gemm_blockscaled(b.qdyT, b.sdyT, fq.ROW_1x128, b.qxT, b.sxT,
                                                                  fq.ROW_1x128, fq.B_NK, c=b.dW),
         "mfma", gemm_flops),
    ]
    group_of = {"quant_transpose x": "quant_transpose", "quant_128x128 W": "quant",
                "quant_transpose dy": "quant_transpose"}

    def step(i):
        b = sets[i % 2]
        for _, fn, _, _ in ops:
            fn(b)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region 1: the whole step, K times, bracketed by synchronizations;
    # no events inside the step
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(i)
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
        b = sets[s % 2]
        ev[s][0].record(stream)
        for i, (_, fn, _, _) in enumerate(ops):
            fn(b)
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
        rec = gemm_rec(work, t * 1e3) if bound == "mfma" else hbm_rec(work, t * 1e3)
        rec["kernel"] = name
        breakdown.append(rec)
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

    # quality monitor of the backward workload (full size): values flushed to
    # zero by the row tiles of dy against its transposed column tiles
    b0 = sets[0]
    step(0)
    torch.cuda.synchronize()
    step_stats = {"underflow_dy_row_tiles": underflow(b0.dy, b0.qdy),
                  "underflow_dy_col_tiles": underflow(b0.dy.t(), b0.qdyT)}

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
        "step_stats": step_stats,
        "wall_s_timed": round(wall, 3),
    }

    if "clock" in parts:
        clk = sustained_clock_mhz(dev, lambda: [step(i) for i in range(10)])
        out["sustained_clock"] = clk
        if clk:
            f = clk["median_mhz"] / PEAK_CLOCK_MHZ
            out["roofline"]["frac_at_measured_clock"] = round(out["roofline"]["frac"] / f, 4)
            out["roofline"]["peak_at_measured_clock"] = round(PEAK_FP8_TFLOPS * f, 1) \
                if dbound == "mfma" else None
    out["hbm_copy_GBps"] = copy_ceiling_gbs(dev)

    if "e4m3" in parts:
        out["fwd_quantize_on_store"] = quantize_on_store(fq, sets, args.steps, stream)
    if "pow2" in parts:
        out["pow2_scales"] = pow2_step(fq, sets, args, stream, gemm_flops)
    if "adam" in parts:
        out["fp8_adam"] = adam_step(fq, sets[0], args, stream)
    del sets
    torch.cuda.empty_cache()
    if "long_k" in parts:
        out["long_k"] = long_k(fq, synthetic, dev, stream)
        torch.cuda.empty_cache()
    if "moe" in parts:
        out["moe_grouped"] = moe_grouped(fq, synthetic, dev, stream)
        torch.cuda.empty_cache()

    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(x_bits, w_bits, dy_bits, args.cpu_rows)
    print(json.dumps(out))


def quantize_on_store(fq, sets, reps, stream):
    """The forward GEMM storing its output quantized (E4M3 codes + 1x128
    scales: the next layer's activation quantization) against the same GEMM
    with bf16 output followed by the separate 1x128 quantization of y."""
    import torch
    qy = [torch.empty((M, N), dtype=torch.uint8, device=b.x.device) for b in sets]
    sy = [torch.empty((M, N // 128), dtype=torch.float32, device=b.x.device) for b in sets]
    res = {}
    for name, mk in (
            ("gemm_bf16_out", lambda i: lambda: fq.fp8_gemm_blockscaled(
                sets[i].qx, sets[i].sx, fq.ROW_1x128, sets[i].qw, sets[i].sw, fq.BLOCK_128x128, fq.B_NK,
                c=sets[i].y)),
            ("quant_1x128_y", lambda i: lambda: fq.fp8_quant_blockwise(sets[i].y, fq.ROW_1x128, q=qy[i], s=sy[i])),
            ("gemm_e4m3_out", lambda i: lambda: fq.fp8_gemm_blockscaled_e4m3(
                sets[i].qx, sets[i].sx, fq.ROW_1x128, sets[i].qw, sets[i].sw, fq.BLOCK_128x128, fq.B_NK,
                out=(qy[i], sy[i])))):
        res[name + "_us"] = round(time_launches([mk(0), mk(1)], reps, stream), 2)
    res["saving_us"] = round(res["gemm_bf16_out_us"] + res["quant_1x128_y_us"] - res["gemm_e4m3_out_us"], 2)
    return res


def pow2_step(fq, sets, args, stream, gemm_flops):
    """The same step with power-of-two scales (E8M0 bytes; the scaled MFMA
    applies them), timed like the main step."""
    import torch
    u8 = torch.uint8
    KB, NB, MB = K // 128, N // 128, M // 128
    dev = sets[0].x.device

    def e8(rows, cols):
        return torch.empty((rows, (cols + 3) // 4 * 4), dtype=u8, device=dev)[:, :cols]
    es = [dict(x=e8(M, KB), w=e8(NB, KB), dy=e8(M, NB), dyT=e8(N, MB), xT=e8(K, MB)) for _ in sets]
    p2_ops = [
        ("quant_transpose x", lambda b, e: fq.fp8_quant_transpose_e8m0(b.x, out=(b.qx, e["x"], b.qxT, e["xT"])),
         M * K * 2 + 2 * M * K + M * KB + K * MB),
        ("quant_128x128 W", lambda b, e: fq.fp8_quant_blockwise_e8m0(b.w, fq.BLOCK_128x128, q=b.qw, e=e["w"]),
         N * K * 2 + N * K + NB * KB),
        ("gemm fwd y=xW^T", lambda b, e: fq.fp8_gemm_e8m0(b.qx, e["x"], b.qw, e["w"], fq.BLOCK_128x128, fq.B_NK,
                                                         c=b.y), None),
        ("quant_transpose dy", lambda b, e: fq.fp8_quant_transpose_e8m0(b.dy, out=(b.qdy, e["dy"], b.qdyT, e["dyT"])),
         M * N * 2 + 2 * M * N + M * NB + N * MB),
        ("gemm dgrad dx=dyW", lambda b, e: fq.fp8_gemm_e8m0(b.qdy, e["dy"], b.qw, e["w"], fq.BLOCK_128x128,
                                                           fq.B_KN, c=b.dx), None),
        ("gemm wgrad dW=dy^T x", lambda b, e: fq.fp8_gemm_e8m0(b.qdyT, e["dyT"], b.qxT, e["xT"], fq.ROW_1x128,
                                                              fq.B_NK, c=b.dW), None),
    ]

    def step(i):
        for _, fn, _ in p2_ops:
            fn(sets[i % 2], es[i % 2])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    p2_step_ms = e0.elapsed_time(e1) / args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(p2_ops) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, (_, fn, _) in enumerate(p2_ops):
            fn(sets[s % 2], es[s % 2])
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    res = {"ms_per_step": round(p2_step_ms, 4),
           "TFLOP/s": round(3 * gemm_flops / (p2_step_ms * 1e-3) / 1e12, 2), "kernels": []}
    for i, (name, _, nbytes) in enumerate(p2_ops):
        us = sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) * 1e3 / args.steps
        rec = gemm_rec(gemm_flops, us) if name.startswith("gemm") else hbm_rec(nbytes, us)
        rec["kernel"] = name
        res["kernels"].append(rec)
    return res


def adam_step(fq, b, args, stream):
    """The optimizer step of the same layer: AdamW with FP8 moments on an
    fp32 master copy of W, the step's fp32 dW as gradient."""
    import torch
    n_w = N * K
    p_w = b.w.float().reshape(-1).contiguous()
    g_w = b.dW.reshape(-1)
    st8 = fq.fp8_adam_state(n_w, b.x.device)
    # warmup on a copy of the state (the timed steps continue from step 1)
    warm = fq.fp8_adam_state(n_w, b.x.device)
    p_warm = p_w.clone()
    settle([lambda: fq.fp8_adam_step(p_warm, g_w, warm, lr=1e-4, weight_decay=0.1, step=1)])
    del warm, p_warm
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
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    # algorithmic bytes: parameters read and written (8), fp32 gradient (4),
    # both moments' codes read and written (4), their scales (16 per 128)
    rec = hbm_rec(n_w * 16 + (n_w // 128) * 16, us)
    rec.update({"params": n_w, "state_bytes_per_param": 2 + 8 / 128})
    return rec


def long_k(fq, synthetic, dev, stream, reps=10, sample=256):
    """Long-K stress: x [16384 x 8192] bf16 with log-normal row magnitudes,
    W [8192 x 8192] bf16 ~N(0, 0.02).  Quantizers (1x128, 128x128, per
    tensor), the 16384 x 8192 x 8192 GEMM with blockwise and with per-tensor
    scales (bf16 out), and with power-of-two tile scales; underflow of x's
    codes and the error of each GEMM against the exact fp64 product of the
    bf16 inputs on `sample` seeded rows."""
    import torch
    Mk, Nk, Kk = 16384, 8192, 8192
    xb, wb = synthetic.long_k(Mk, Nk, Kk)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(dev)
    w = [torch.from_numpy(wb.view(np.int16)).view(torch.bfloat16).to(dev) for _ in range(2)]
    del xb, wb
    KBk, NBk = Kk // 128, Nk // 128
    u8, f32 = torch.uint8, torch.float32
    qx, sx = torch.empty((Mk, Kk), dtype=u8, device=dev), torch.empty((Mk, KBk), dtype=f32, device=dev)
    qxt, sxt = torch.empty((Mk, Kk), dtype=u8, device=dev), torch.empty((1, 1), dtype=f32, device=dev)
    qw = [torch.empty((Nk, Kk), dtype=u8, device=dev) for _ in range(2)]
    sw = [torch.empty((NBk, KBk), dtype=f32, device=dev) for _ in range(2)]
    qwt = [torch.empty((Nk, Kk), dtype=u8, device=dev) for _ in range(2)]
    swt = [torch.empty((1, 1), dtype=f32, device=dev) for _ in range(2)]
    y = torch.empty((Mk, Nk), dtype=torch.bfloat16, device=dev)
    flops = 2.0 * Mk * Nk * Kk
    bx, bw = Mk * Kk, Nk * Kk
    res = {"shape": {"M": Mk, "N": Nk, "K": Kk}}
    res["quant_1x128 x"] = hbm_rec(3 * bx + 4 * Mk * KBk, time_launches(
        [lambda: fq.fp8_quant_blockwise(x, fq.ROW_1x128, q=qx, s=sx)], reps, stream))
    res["quant_tensor x"] = hbm_rec(5 * bx, time_launches(
        [lambda: fq.fp8_quant_blockwise(x, fq.TENSOR, q=qxt, s=sxt)], reps, stream))
    res["quant_128x128 W"] = hbm_rec(3 * bw + 4 * NBk * KBk, time_launches(
        [lambda i=i: fq.fp8_quant_blockwise(w[i], fq.BLOCK_128x128, q=qw[i], s=sw[i]) for i in range(2)],
        reps, stream))
    res["quant_tensor W"] = hbm_rec(5 * bw, time_launches(
        [lambda i=i: fq.fp8_quant_blockwise(w[i], fq.TENSOR, q=qwt[i], s=swt[i]) for i in range(2)],
        reps, stream))
    res["gemm blockwise"] = gemm_rec(flops, time_launches(
        [lambda i=i: fq.fp8_gemm_blockscaled(qx, sx, fq.ROW_1x128, qw[i], sw[i], fq.BLOCK_128x128, fq.B_NK, c=y)
         for i in range(2)], reps, stream))
    res["gemm per-tensor"] = gemm_rec(flops, time_launches(
        [lambda i=i: fq.fp8_gemm_blockscaled(qxt, sxt, fq.TENSOR, qwt[i], swt[i], fq.TENSOR, fq.B_NK, c=y)
         for i in range(2)], reps, stream))
    ex = torch.empty((Mk, KBk), dtype=u8, device=dev)
    ew = torch.empty((NBk, KBk), dtype=u8, device=dev)
    qx2, qw2 = torch.empty_like(qx), torch.empty_like(qw[0])
    fq.fp8_quant_blockwise_e8m0(x, fq.ROW_1x128, q=qx2, e=ex)
    fq.fp8_quant_blockwise_e8m0(w[0], fq.BLOCK_128x128, q=qw2, e=ew)
    res["gemm pow2"] = gemm_rec(flops, time_launches(
        [lambda: fq.fp8_gemm_e8m0(qx2, ex, qw2, ew, fq.BLOCK_128x128, fq.B_NK, c=y)], reps, stream))

    # quality: underflow of x's codes; error against the exact product
    rows = torch.from_numpy(synthetic.sample_rows(Mk, sample, 503)).to(dev)
    exact = x.index_select(0, rows).double() @ w[0].double().t().contiguous()
    yf = torch.empty((Mk, Nk), dtype=f32, device=dev)

    def errors(run):
        run()
        got = yf.index_select(0, rows).double()
        d = got - exact
        return {"frobenius": float(d.norm() / exact.norm()),
                "mean_row": float((d.norm(dim=1) / exact.norm(dim=1)).mean())}
    quality = {
        "blockwise": errors(lambda: fq.fp8_gemm_blockscaled(qx, sx, fq.ROW_1x128, qw[0], sw[0], fq.BLOCK_128x128,
                                                            fq.B_NK, c=yf)),
        "per_tensor": errors(lambda: fq.fp8_gemm_blockscaled(qxt, sxt, fq.TENSOR, qwt[0], swt[0], fq.TENSOR,
                                                             fq.B_NK, c=yf)),
        "pow2": errors(lambda: fq.fp8_gemm_e8m0(qx2, ex, qw2, ew, fq.BLOCK_128x128, fq.B_NK, c=yf)),
    }
    quality["blockwise"]["underflow_x"] = underflow(x, qx)
    quality["per_tensor"]["underflow_x"] = underflow(x, qxt)
    quality["pow2"]["underflow_x"] = underflow(x, qx2)
    quality["sampled_rows"] = sample
    res["quality"] = quality
    return res


def moe_grouped(fq, synthetic, dev, stream, reps=10):
    """Grouped MoE GEMMs on the seeded MoE workload of the parity tests:
    8192 tokens, hidden 2048, 128 experts of intermediate 768, top-8 Zipf(1.1)
    routing, groups padded to 128 rows.  For each expert layer the forward
    (bf16 out), the forward stored quantized (E4M3 codes + 1x128 scales, set
    against the bf16 forward plus a separate 1x128 quantization of its
    output), the backward's dgrad (expert weight read as stored, bf16 out)
    and wgrad (per-expert token ranges, transposed re-quantized operands,
    fp32 out).  TFLOP/s count the real (unpadded) rows only; `frac_attainable`
    is max(t_MFMA, t_HBM) / time, with t_MFMA the real FLOPs at the FP8 peak
    and t_HBM the launch's algorithmic bytes at the HBM peak."""
    import torch
    m = synthetic.moe()
    dgu, dd = synthetic.moe_backward_dy(m)
    G = m.w_gate_up.shape[0]
    M_pad = int(m.offsets[-1])
    real = int(m.counts.sum())
    off = torch.from_numpy(m.offsets.astype(np.int32)).to(dev)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    out = {"tokens": int(m.x.shape[0]), "experts": G, "topk": 8, "real_rows": real, "M_pad": M_pad,
           "largest_group": int(m.counts.max()), "smallest_group": int(m.counts.min())}
    for name, a_bits, w_bits, dy_bits in (("gate_up", m.a_gate_up, m.w_gate_up, dgu),
                                          ("down", m.a_down, m.w_down, dd)):
        Nn, Kk = w_bits.shape[1], w_bits.shape[2]
        a = bf(a_bits)
        w = bf(w_bits.reshape(G * Nn, Kk))
        dy = bf(dy_bits)
        qa, sa = fq.fp8_quant_blockwise(a, fq.ROW_1x128)
        qw, sw = fq.fp8_quant_blockwise(w, fq.BLOCK_128x128)
        qw = qw.view(G, Nn, Kk)
        sw = sw.view(G, Nn // 128, -(-Kk // 128))
        qdy, sdy, qdyT, sdyT = fq.fp8_quant_transpose(dy)
        _, _, qaT, saT = fq.fp8_quant_transpose(a, rows_out=False)
        c = torch.empty((M_pad, Nn), dtype=torch.bfloat16, device=dev)
        dx = torch.empty((M_pad, Kk), dtype=torch.bfloat16, device=dev)
        dw = torch.empty((G, Nn, Kk), dtype=torch.float32, device=dev)
        qc = torch.empty((M_pad, Nn), dtype=torch.uint8, device=dev)
        sc = torch.empty((M_pad, -(-Nn // 128)), dtype=torch.float32, device=dev)
        flops = 2.0 * real * Nn * Kk
        kb, nb = -(-Kk // 128), -(-Nn // 128)
        wbytes = G * Nn * Kk + G * nb * kb * 4
        nbytes = {
            "fwd": M_pad * Kk + M_pad * kb * 4 + wbytes + M_pad * Nn * 2,
            "fwd_e4m3": M_pad * Kk + M_pad * kb * 4 + wbytes + M_pad * Nn + M_pad * nb * 4,
            "dgrad": M_pad * Nn + M_pad * nb * 4 + wbytes + M_pad * Kk * 2,
            "wgrad": (Nn + Kk) * M_pad + (Nn + Kk) * (M_pad // 128) * 4 + G * Nn * Kk * 4,
        }
        res = {"N": Nn, "K": Kk}
        for part, fn in (("fwd", lambda: fq.fp8_grouped_gemm(qa, sa, off, qw, sw, c=c)),
                         ("fwd_e4m3", lambda: fq.fp8_grouped_gemm_e4m3(qa, sa, off, qw, sw, q=qc, s=sc)),
                         ("dgrad", lambda: fq.fp8_grouped_gemm_dgrad(qdy, sdy, off, qw, sw, c=dx)),
                         ("wgrad", lambda: fq.fp8_grouped_gemm_wgrad(qdyT, sdyT, qaT, saT, off, c=dw))):
            us = time_launches([fn], reps, stream)
            rec = gemm_rec(flops, us)
            t_mfma = flops / (PEAK_FP8_TFLOPS * 1e12) * 1e6
            t_hbm = nbytes[part] / (PEAK_HBM_GBS * 1e9) * 1e6
            rec.update({"algorithmic_bytes": int(nbytes[part]), "t_mfma_us": round(t_mfma, 1),
                        "t_hbm_us": round(t_hbm, 1), "frac_attainable": round(max(t_mfma, t_hbm) / us, 4)})
            res[part] = rec
        q_us = time_launches([lambda: fq.fp8_quant_blockwise(c, fq.ROW_1x128, q=qc, s=sc)], reps, stream)
        res["quant_1x128_fwd_out_us"] = round(q_us, 2)
        res["e4m3_saving_us"] = round(res["fwd"]["us"] + q_us - res["fwd_e4m3"]["us"], 2)
        out[name] = res
        del a, w, dy, qa, sa, qw, sw, qdy, sdy, qdyT, sdyT, qaT, saT, c, dx, dw, qc, sc
    return out


def cpu_baseline(x_bits, w_bits, dy_bits, rows_per_gemm):
    """The oracle on a bounded sample of the same step: full-tensor quantizers
    for x (1x128) and W (128x128) and the three GEMMs on `rows_per_gemm`
    output rows each; reported as GEMM TFLOP/s of the sample, with all host
    threads, and with one thread on a smaller sample."""
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
    threads = oracle.num_threads()
    # one thread: the forward GEMM on 32 rows and the 1x128 quantizer of x
    oracle.set_num_threads(1)
    try:
        r1 = synthetic.sample_rows(M, 32, 9)
        t1 = time.perf_counter()
        oracle.gemm_blockscaled(qx, sx, "row", qw, sw, "block", "NK", rows=r1)
        t1 = time.perf_counter() - t1
        tq1 = time.perf_counter()
        oracle.quant_1x128(xf)
        tq1 = time.perf_counter() - tq1
    finally:
        oracle.set_num_threads(threads)
    return {"value": round(flops / t_g / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": "quant 1x128 x + 128x128 W (full tensors, %.1f GB/s), quant+transpose of dy and x "
                      "(full, %.2f s), and fwd/dgrad GEMMs on all %d rows, wgrad on %d sampled rows "
                      "(%.2f s); value = GEMM FLOPs of the sample / GEMM time"
                      % (q_bytes / t_q / 1e9, t_t, len(rows), len(rows_w), t_g),
            "single_thread": {"gemm_TFLOP/s": round(2.0 * len(r1) * N * K / t1 / 1e12, 6),
                              "quant_1x128_GB/s": round(xf.size * 3 / tq1 / 1e9, 3),
                              "sample": "fwd GEMM on 32 rows; 1x128 quantizer on all of x"},
            "total_s": round(time.perf_counter() - t0, 2)}


if __name__ == "__main__":
    main()
