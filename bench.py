"""Benchmark of the fused 4-bit + LoRA linear layer (forward + backward) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--m M]

A step is one forward (qlin_fwd) plus one backward (qlin_bwd: dX, dA, dB) of
one layer over one batch of synthetic tokens, with inputs resident in HBM.
The frozen weight is quantized once before timing, as in training.  For the
weight-streaming (few-token) workloads the step cycles through enough
distinct packed-weight copies (> 2x the 256 MB Infinity Cache) that every
step streams its weight from HBM, as a real multi-layer model does.

Prints one JSON line.  ``value`` is the weight-stream rate (packed-weight
bytes read per step, forward + backward, / step time) for HBM-bound
workloads and TFLOP/s for MFMA-bound ones.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused 4-bit+LoRA linear fwd+bwd TFLOP/s & weight GB/s, % of roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
MALL_BYTES = 256 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="q_proj")
    p.add_argument("--m", type=int, default=None, help="token count override")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel-iters", type=int, default=200)
    p.add_argument("--eager", action="store_true",
                   help="launch kernels directly instead of replaying a HIP graph "
                        "(for counter collection, which profiles eager dispatches)")
    p.add_argument("--calibrate-copy-mb", type=int, default=0,
                   help="before timing, copy a buffer of this many MiB once: a plain copy "
                        "kernel of known size that scales the HBM byte counters")
    return p.parse_args()


# Kernel sources whose HBM byte counts a committed traffic record refers to.
TRAFFIC_SOURCES = {
    "k_gemv_fwd": ("quantized_base_rank_amd/csrc/gemv_fwd.hip",
                   "quantized_base_rank_amd/csrc/device_common.hpp"),
    "k_fwd_gemm": ("quantized_base_rank_amd/csrc/fwd_gemm.hip",
                   "quantized_base_rank_amd/csrc/device_common.hpp"),
}


def source_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy of known size), taken from the record
    under profiles/; None when there is no record or the kernel's source has
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import quantized_base_rank_amd as qb
    from quantized_base_rank_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    if args.m is not None:
        wl = wl.with_m(args.m)
    elif args.workload == "q_proj":
        wl = wl.with_m(16)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(wl, seed=0)

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def quantize(Wt):
        if wl.fmt == "nf4":
            return qb.qlin_quantize_nf4(Wt, wl.block, wl.dq_block)
        return qb.qlin_quantize_int4_group(Wt, wl.block)

    hbm_bound = wl.M <= 16
    wbytes = wl.packed_weight_bytes()
    n_copies = max(1, math.ceil(2 * MALL_BYTES / wbytes) + 1) if hbm_bound else 1
    t0 = time.time()
    weights = [quantize(torch.from_numpy(inp.W).to(dev))]
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    for _ in range(1, n_copies):
        Wt = torch.randn((wl.d_out, wl.d_in), generator=g, device=dev, dtype=torch.float32) * 0.02
        weights.append(quantize(Wt))
        del Wt
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    if args.calibrate_copy_mb > 0:
        nb = args.calibrate_copy_mb << 20
        src = torch.ones(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    x, A, B, dy = (dev_bf16(a) for a in (inp.x, inp.A, inp.B, inp.dy))
    r, s, pool = wl.r, wl.s, wl.pool
    ws = qb.workspace(dev, qb.qlin_workspace_bytes(weights[0], wl.M, r, pool))
    y = torch.empty((wl.M, wl.d_out), dtype=torch.bfloat16, device=dev)
    u = torch.empty((wl.M, r), dtype=torch.float32, device=dev)
    dx = torch.empty((wl.M, wl.d_in), dtype=torch.bfloat16, device=dev)
    dA = torch.empty((r, wl.k_a), dtype=torch.bfloat16, device=dev)
    dB = torch.empty((wl.d_out, r), dtype=torch.bfloat16, device=dev)

    def step(i):
        w = weights[i % n_copies]
        qb.qlin_fwd(w, x, A, B, r, s, pool, y=y, u_out=u, ws=ws)
        qb.qlin_bwd(w, x, A, B, r, s, dy, pool, u_saved=u, dx=dx, dA=dA, dB=dB, ws=ws)

    def fwd_only(i):
        qb.qlin_fwd(weights[i % n_copies], x, A, B, r, 0.0, pool, y=y, u_out=None, ws=ws,
                    want_u=False)

    class Eager:
        def __init__(self, fn, n, offset):
            self.fn, self.n, self.offset = fn, n, offset

        def replay(self):
            for i in range(self.n):
                self.fn(self.offset + i)

    def capture(fn, n, offset=0):
        """One HIP graph holding exactly n calls of fn (host launch cost is
        paid once at capture, not in the timed region)."""
        if args.eager:
            return Eager(fn, n, offset)
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            fn(offset)  # eager warm call outside the capture
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(offset + i)
        return g

    def timed(g):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    if args.warmup > 0:
        gw = capture(step, args.warmup)
        gw.replay()
        torch.cuda.synchronize()
    gt = capture(step, args.steps, offset=args.warmup)
    ms_per_step = timed(gt) / args.steps

    flops = wl.flops_fwd() + wl.flops_bwd()
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    weight_gbs = 2 * wbytes / (ms_per_step * 1e-3) / 1e9

    # dominant kernel timed alone on the stream it runs on: the forward with the
    # adapter off and no u is exactly one launch of the weight-streaming (few
    # tokens) or the MFMA kernel.
    kit = args.kernel_iters
    gk = capture(fwd_only, kit)
    gk.replay()
    k_ms = timed(gk) / kit
    if hbm_bound:
        k_bytes = wbytes + wl.M * wl.d_in * 2 + wl.M * wl.d_out * 2
        achieved = k_bytes / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic("k_gemv_fwd", args.workload),
                "kernel": "k_gemv_fwd", "bytes_per_launch": k_bytes,
                "avg_launch_us": round(k_ms * 1e3, 3)}
        value, unit = weight_gbs, "GB/s"
    else:
        k_flops = 2 * wl.M * wl.d_out * wl.d_in
        achieved = k_flops / (k_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": recorded_traffic("k_fwd_gemm", args.workload),
                "kernel": "k_fwd_gemm", "flops_per_launch": k_flops,
                "avg_launch_us": round(k_ms * 1e3, 3)}
        value, unit = tflops, "TFLOP/s"

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "d_out": wl.d_out, "d_in": wl.d_in, "M": wl.M, "r": wl.r,
                   "s": wl.s, "format": wl.fmt, "block": wl.block, "dq_block": wl.dq_block,
                   "pool": wl.pool, "weight_copies": n_copies},
        "tflops": round(tflops, 3), "weight_gbs": round(weight_gbs, 1),
        "packed_weight_bytes": wbytes, "flops_per_step": flops,
        "roofline": roof, "setup_s": round(setup_s, 2),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, hbm_bound, wbytes, flops)
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, inp, hbm_bound, wbytes, flops):
    """The CPU oracle (float64 numpy) on a bounded sample of the same layer."""
    import numpy as np

    from oracle import qlin_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    # sample: the whole layer when it is small; otherwise the first rows of W
    # and a proportional share of the work
    rows = wl.d_out if wl.d_out * wl.d_in <= (1 << 24) else max(256, (1 << 24) // wl.d_in)
    M = min(wl.M, 256)
    W = inp.W[:rows]
    t0 = time.time()
    if wl.fmt == "nf4":
        codes, am, am2 = O.quantize_nf4(W, wl.block, wl.dq_block)
    else:
        codes, sc, zp = O.quantize_int4_group(W, wl.block)
    tq = time.time() - t0
    xf = O.bf16_bits_to_f64(inp.x[:M])
    Af = O.bf16_bits_to_f64(inp.A)
    Bf = O.bf16_bits_to_f64(inp.B[:rows])
    dyf = O.bf16_bits_to_f64(inp.dy[:M, :rows])
    n_steps, t_steps = 0, 0.0
    while t_steps < 10.0 and n_steps < 50:
        t0 = time.time()
        if wl.fmt == "nf4":
            Wd = O.bf16_bits_to_f64(O.dequant_nf4_bf16(codes, am, am2, wl.block, wl.dq_block))
        else:
            Wd = O.bf16_bits_to_f64(O.dequant_int4_bf16(codes, sc, zp, wl.block))
        y, u = O.lora_forward(Wd, xf, Af, Bf, wl.s, wl.pool)
        O.lora_backward(Wd, xf, Af, Bf, wl.s, dyf, wl.pool, u=u)
        t_steps += time.time() - t0
        n_steps += 1
    sec = t_steps / n_steps
    frac = (rows / wl.d_out) * (M / wl.M)
    if hbm_bound:
        val = 2 * wbytes * (rows / wl.d_out) / sec / 1e9
        unit = "GB/s"
    else:
        val = flops * frac / sec / 1e12
        unit = "TFLOP/s"
    return {"value": round(val, 6), "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{rows} of {wl.d_out} weight rows, {M} of {wl.M} tokens; float64 numpy "
                      f"dequant + forward + backward, {n_steps} steps averaged; quantize {tq:.2f} s",
            "sec_per_sample_step": round(sec, 4)}


if __name__ == "__main__":
    main()
