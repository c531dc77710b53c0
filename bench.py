"""Benchmark of the fused 4-bit + LoRA linear layer (forward + backward) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--m M]

A step is one forward (qlin_fwd: y and u) plus one backward (qlin_bwd: dX,
dA, dB) of one layer over one batch of synthetic tokens, with every input
resident in HBM.  The frozen weight is quantized once before timing, as in
training.  The default workload is the LLaMA-2-70B MLP down_proj at its real
shape (W 8192 x 28672 NF4 + double quantization, LoRA r = 64, 4096 tokens),
the largest single-GPU configuration; ``value`` is then TFLOP/s of the whole
step (fwd 2MNK + 2MKr + 2MNr, bwd 2MNK + 4MNr + 4MKr; dequantization counts
as zero).  Few-token workloads (M <= 16) are HBM-bound: their steps cycle
through enough distinct packed-weight copies (> 2x the 256 MB Infinity
Cache) that every step streams its weight from HBM, and ``value`` is the
weight-stream rate (2 x packed-weight bytes per step / step time).

``roofline`` describes the step's dominant kernel as the step launches it:
its average device duration, measured with HIP events that the library
records on the launch stream right around that kernel's launch (large M:
inside every timed step; few tokens, whose steps are timed as a replayed
graph: in as many eagerly run steps, each queued behind a spin kernel so that
the events bracket the kernel and not host launch gaps), against its
algorithmic flops (MFMA-bound) or bytes (HBM-bound) per launch.

Prints one JSON line.
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
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="down_proj70b")
    p.add_argument("--m", type=int, default=None, help="token count override")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--lq", action="store_true",
                   help="time the low-rank plus quantized decomposition (qlin_lq_nf4) of the "
                        "workload's weight instead of the layer step")
    p.add_argument("--lq-iters", type=int, default=2)
    p.add_argument("--lq-power", type=int, default=1)
    p.add_argument("--kernel-iters", type=int, default=200,
                   help="few-token workloads: graph-replayed launches for the kernel timing")
    p.add_argument("--reference-gemm", action="store_true",
                   help="time hipBLASLt's bf16 GEMMs (torch.matmul on a materialised bf16 W, which the layer "
                        "never makes) at the workload's forward and input-gradient shapes, as a reference "
                        "point for the MFMA roofline; prints its own JSON line")
    p.add_argument("--calibrate-copy-mb", type=int, default=0,
                   help="before timing, copy a buffer of this many MiB once: a plain copy "
                        "kernel of known size that scales the HBM byte counters")
    return p.parse_args()


# Kernel sources whose HBM byte counts a committed traffic record refers to.
TRAFFIC_SOURCES = {
    "k_gemv_fwd": ("quantized_base_rank_amd/csrc/gemv_fwd.hip",),
    "k_gemv_dx": ("quantized_base_rank_amd/csrc/gemv_dx.hip",),
    "k_gemv_fwd_stream": ("quantized_base_rank_amd/csrc/gemv_stream.hip",),
    "k_gemv_dx_stream": ("quantized_base_rank_amd/csrc/gemv_dx_stream.hip",),
    "k_fwd_gemm": ("quantized_base_rank_amd/csrc/fwd_gemm.hip",),
    "k_dx_gemm": ("quantized_base_rank_amd/csrc/dx_gemm.hip",),
}
COMMON_SOURCES = ("quantized_base_rank_amd/csrc/device_common.hpp",)


def source_digest(kernel):
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES[kernel] + COMMON_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload, m=None):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy of known size), taken from the record
    under profiles/ (named for the token count too when it is not the
    workload's own); None when there is no record or the kernel's source has
    changed since the counters were taken."""
    suffix = f"_M{m}" if m is not None else ""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}{suffix}.txt")
    try:
        with open(path) as f:
            text = f.read()
        rec = json.loads(text[text.index("{"):text.rindex("}") + 1])
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec.get("traffic_bytes_per_launch")


def kernel_work(wl, kernel):
    """Algorithmic work of one launch of `kernel` in a step of `wl`:
    (amount, 'flop' | 'byte')."""
    M, N, K, r, Ka = wl.M, wl.d_out, wl.d_in, wl.r, wl.k_a
    wbytes = wl.packed_weight_bytes()
    if kernel == "k_fwd_gemm":        # x W^T plus the appended adapter term
        return 2 * M * N * K + 2 * M * N * r, "flop"
    if kernel == "k_dx_gemm":         # dY W plus the appended du A term
        return 2 * M * N * K + 2 * M * Ka * r, "flop"
    if kernel == "k_gemv_fwd":        # W, x, A (fused u), B, y, u
        return wbytes + 2 * M * K + 2 * r * Ka + 2 * N * r + 2 * M * N + 4 * M * r, "byte"
    if kernel == "k_gemv_dx":         # W, dY, x, dX, A, B, u, dA, dB
        return (wbytes + 2 * M * N + 4 * M * K + 4 * r * Ka + 4 * N * r + 4 * M * r), "byte"
    if kernel == "k_gemv_fwd_stream":  # W, x, B, u, y
        return wbytes + 2 * M * K + 2 * N * r + 4 * M * r + 2 * M * N, "byte"
    if kernel == "k_gemv_dx_stream":  # W, dY, A, du, dX; unpooled also x and dA
        extra = 2 * M * K + 2 * r * K if wl.pool == 1 else 0
        return wbytes + 2 * M * N + 2 * r * Ka + 4 * M * r + 2 * M * K + extra, "byte"
    raise KeyError(kernel)


def streamed(wl):
    """Few-token layers on weights above 32 M elements run the streamed
    forward and input-gradient kernels (the library's own rule)."""
    return wl.M <= 16 and wl.d_out * wl.d_in > (1 << 25)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer benchmark runs on exactly one GPU; --gpus must be 1",
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
    if args.lq:
        return lq_main(args, wl, inp, qb, torch, np, dev)
    if args.reference_gemm:
        return reference_gemm_main(args, wl, inp, torch, np, dev)

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def quantize(Wt):
        if wl.fmt == "nf4":
            return qb.qlin_quantize_nf4(Wt, wl.block, wl.dq_block)
        if wl.fmt == "nf":
            return qb.qlin_quantize_nf(Wt, wl.bits, wl.block, wl.dq_block)
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

    def fwd(i):
        qb.qlin_fwd(weights[i % n_copies], x, A, B, r, s, pool, y=y, u_out=u, ws=ws)

    def bwd(i):
        qb.qlin_bwd(weights[i % n_copies], x, A, B, r, s, dy, pool, u_saved=u, dx=dx, dA=dA,
                    dB=dB, ws=ws)

    def step(i):
        fwd(i)
        bwd(i)

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record()   # creates the device event, so its handle can be passed on
        return e

    def capture(fn, n, offset=0):
        """One HIP graph holding exactly n calls of fn (host launch cost is
        paid once at capture, not in the timed region)."""
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            fn(offset)  # eager warm call outside the capture
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(n):
                fn(offset + i)
        return gr

    def timed_graph(gr):
        e0, e1 = new_event(), new_event()
        torch.cuda.synchronize()
        e0.record()
        gr.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def hooked_ms(name, i, lead_cycles):
        """GPU time of kernel `name` as step i launches it: events recorded by
        the library right around that launch.  A spin kernel queued first keeps
        the GPU busy while the host queues the whole step, so the events
        bracket the kernel alone and not host launch gaps."""
        ev = (new_event(), new_event())
        if lead_cycles:
            torch.cuda._sleep(lead_cycles)
        qb.qlin_profile_next_launch(name, *ev)
        step(i)
        return ev

    kernel_ms = {}
    if hbm_bound:
        # few tokens: each step is tens to hundreds of microseconds, so the
        # step time comes from a captured graph of steps; the kernels are
        # timed by events the library records around their launch in
        # eagerly run steps.
        if args.warmup > 0:
            gw = capture(step, args.warmup)
            gw.replay()
            torch.cuda.synchronize()
        gt = capture(step, args.steps, offset=args.warmup)
        ms_per_step = timed_graph(gt) / args.steps
        cands = ("k_gemv_fwd_stream", "k_gemv_dx_stream") if streamed(wl) else ("k_gemv_fwd", "k_gemv_dx")
        lead = 2_000_000  # ~1 ms of spinning at the shader clock
        for name in cands:
            ev = hooked_ms(name, 0, lead)
            torch.cuda.synchronize()
            kernel_ms[name] = ev[0].elapsed_time(ev[1])
        dominant = max(kernel_ms, key=kernel_ms.get)
        evs = [hooked_ms(dominant, args.warmup + i, lead) for i in range(args.steps)]
        torch.cuda.synchronize()
        k_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
        timing = "eager steps after a spin kernel; kernel bracketed by events inside each step"
    else:
        # large M: milliseconds per step, launched directly.  After warm-up,
        # one further step per candidate times that candidate; in every timed
        # step the library records events around the dominant kernel's launch.
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        for name in ("k_fwd_gemm", "k_dx_gemm"):
            ev = (new_event(), new_event())
            qb.qlin_profile_next_launch(name, *ev)
            step(0)
            torch.cuda.synchronize()
            kernel_ms[name] = ev[0].elapsed_time(ev[1])
        dominant = max(kernel_ms, key=kernel_ms.get)
        evs = [(new_event(), new_event()) for _ in range(args.steps)]
        e0, e1 = new_event(), new_event()
        torch.cuda.synchronize()
        e0.record()
        for i in range(args.steps):
            qb.qlin_profile_next_launch(dominant, *evs[i])
            step(args.warmup + i)
        e1.record()
        torch.cuda.synchronize()
        ms_per_step = e0.elapsed_time(e1) / args.steps
        k_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
        timing = "launched directly; kernel bracketed by events inside each timed step"

    flops = wl.flops_fwd() + wl.flops_bwd()
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    weight_gbs = 2 * wbytes / (ms_per_step * 1e-3) / 1e9

    work, kind = kernel_work(wl, dominant)
    if kind == "byte":
        achieved = work / (k_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(dominant, args.workload, wl.M if wl.M != WORKLOADS[args.workload].M else None),
                "kernel": dominant, "bytes_per_launch": work}
        value, unit = weight_gbs, "GB/s"
    else:
        achieved = work / (k_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": recorded_traffic(dominant, args.workload, wl.M if wl.M != WORKLOADS[args.workload].M else None),
                "kernel": dominant, "flops_per_launch": work}
        value, unit = tflops, "TFLOP/s"
    roof["avg_launch_us"] = round(k_ms * 1e3, 3)
    roof["timing"] = timing
    roof["candidates_us"] = {k: round(v * 1e3, 3) for k, v in kernel_ms.items()}

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "d_out": wl.d_out, "d_in": wl.d_in, "M": wl.M, "r": wl.r,
                   "s": wl.s, "format": wl.fmt, "bits": wl.bits, "block": wl.block,
                   "dq_block": wl.dq_block, "pool": wl.pool, "weight_copies": n_copies},
        "tflops": round(tflops, 3), "weight_gbs": round(weight_gbs, 1),
        "frac_of_bf16_peak_step": round(tflops / BF16_PEAK_TFLOPS, 4),
        "packed_weight_bytes": wbytes, "flops_per_step": flops,
        "roofline": roof, "setup_s": round(setup_s, 2),
        "footprint": footprint(wl, wbytes),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, inp, hbm_bound, wbytes, flops)
    print(json.dumps(out), flush=True)


def footprint(wl, wbytes):
    """The pages' memory-footprint claims as context, from this format's own
    bytes: bits per parameter of the packed weight (codes + block constants),
    and what that makes the frozen weights of the models the pages name (the
    QLoRA explainer fine-tunes a 65B model on one 48 GB GPU; the LQ-LoRA
    abstract puts a 2.75-bit LLaMA-2-70B in 27 GB).  NormalFloat-3 with
    double quantization (3.127 bits) is the format of this library nearest
    to that 2.75-bit average, which the pages reach by mixing bit widths."""
    bpp = 8 * wbytes / (wl.d_out * wl.d_in)
    nf3 = 3 + 8 / 64 + 32 / (64 * 256)
    return {"bits_per_param": round(bpp, 4),
            "weights_65b_gb": round(65e9 * bpp / 8 / 1e9, 1),
            "weights_70b_gb": round(70e9 * bpp / 8 / 1e9, 1),
            "weights_70b_nf3_dq_gb": round(70e9 * nf3 / 8 / 1e9, 1),
            "pages": "65B model fine-tuned on one 48 GB GPU (QLoRA); 2.75-bit LLaMA-2-70B in 27 GB (LQ-LoRA)"}


def lq_flops(N, K, r, iters, power):
    """fp32 flops of the decomposition's products: per iteration the range
    and coordinate products (2 N K r each, 2 + 2 power of them), the
    orthonormalisations (two CholeskyQR passes of a Gram and an apply,
    4 r^2 L each) and, after the first, W - U C (2 N K r)."""
    per = (2 + 2 * power) * 2 * N * K * r + (1 + power) * 2 * 4 * r * r * N + power * 2 * 4 * r * r * K
    return iters * per + (iters - 1) * 2 * N * K * r


def reference_gemm_main(args, wl, inp, torch, np, dev):
    """The library's two large products as plain bf16 GEMMs through
    torch.matmul (hipBLASLt) on a materialised bf16 copy of W: y = x W^T
    (W used transposed, as the forward reads it) and dX = dY W.  Not part of
    the layer (which never materialises W): a measured reference point for
    what a dense bf16 GEMM of these shapes reaches on this GPU."""
    M, N, K = wl.M, wl.d_out, wl.d_in
    Wb = torch.from_numpy(np.ascontiguousarray(inp.W, dtype=np.float32)).to(dev).to(torch.bfloat16)
    x = torch.from_numpy(np.ascontiguousarray(inp.x).view(np.int16)).view(torch.bfloat16).to(dev)
    dy = torch.from_numpy(np.ascontiguousarray(inp.dy).view(np.int16)).view(torch.bfloat16).to(dev)
    res = {}
    for name, f in (("x_Wt", lambda: torch.matmul(x, Wb.t())), ("dY_W", lambda: torch.matmul(dy, Wb))):
        for _ in range(max(args.warmup, 1)):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / args.steps * 1e3
        tf = 2 * M * N * K / (us * 1e-6) / 1e12
        res[name] = {"us": round(us, 1), "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    print(json.dumps({"reference": "hipBLASLt bf16 GEMM via torch.matmul (materialised bf16 W)",
                      "config": {"workload": wl.name, "M": M, "N": N, "K": K}, "steps": args.steps,
                      "warmup": args.warmup, **res}), flush=True)


def lq_main(args, wl, inp, qb, torch, np, dev):
    N, K, r = wl.d_out, wl.d_in, wl.r
    W = torch.from_numpy(np.ascontiguousarray(inp.W, dtype=np.float32)).to(dev)
    om_np = np.random.default_rng(1).standard_normal((r, K)).astype(np.float32)
    om = torch.from_numpy(om_np).to(dev)
    for _ in range(max(args.warmup, 1)):
        qb.qlin_lq_nf4(W, r, args.lq_iters, args.lq_power, om)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        _, _, _, errs = qb.qlin_lq_nf4(W, r, args.lq_iters, args.lq_power, om)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = lq_flops(N, K, r, args.lq_iters, args.lq_power)
    out = {"metric": "low-rank plus quantized decomposition (NF4 + rank r), fp32 TFLOP/s",
           "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_decomposition": round(ms, 3),
           "higher_is_better": True, "dtype": "f32", "data": "synthetic",
           "config": {"workload": wl.name, "d_out": N, "d_in": K, "r": r, "iters": args.lq_iters,
                      "power": args.lq_power, "format": "nf4", "block": 64, "dq_block": 256},
           "flops_per_decomposition": flops, "errors": [round(float(e), 6) for e in errs.cpu().numpy()],
           "peak_fp32_tflops": 157.3,
           "frac_of_fp32_peak": round(flops / (ms * 1e-3) / 1e12 / 157.3, 4)}
    if not args.no_cpu_baseline:
        from oracle import qlin_oracle as O
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:  # pragma: no cover
            cores = os.cpu_count() or 1
        rows = 512
        t0 = time.time()
        O.lq_decompose(inp.W[:rows].astype(np.float64), r, args.lq_iters, args.lq_power, om_np)
        sec = time.time() - t0
        out["cpu_baseline"] = {"value": round(lq_flops(rows, K, r, args.lq_iters, args.lq_power) / sec / 1e12, 6),
                               "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
                               "sample": f"the first {rows} rows of W ({rows}x{K}), same r, iterations, "
                                         f"power steps and start; {sec:.2f} s"}
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, inp, hbm_bound, wbytes, flops):
    """The CPU oracle (float64 numpy) on a bounded sample of the same layer."""
    from oracle import qlin_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    # sample: the whole layer when it is small; otherwise the first rows of W
    # (whole double-quantization groups) and a proportional share of the work
    rows = wl.d_out if wl.d_out * wl.d_in <= (1 << 24) else max(256, (1 << 24) // wl.d_in // 4 * 4)
    M = min(wl.M, 256)
    W = inp.W[:rows]
    t0 = time.time()
    if wl.fmt == "nf4":
        codes, am, am2 = O.quantize_nf4(W, wl.block, wl.dq_block)
    elif wl.fmt == "nf":
        codes, am, am2 = O.quantize_nf(W, wl.bits, wl.block, wl.dq_block)
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
        elif wl.fmt == "nf":
            Wd = O.bf16_bits_to_f64(O.dequant_nf_bf16(codes, am, am2, wl.bits, wl.block,
                                                      wl.dq_block))
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
