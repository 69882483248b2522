"""Benchmark: fused linear cross-entropy forward+backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--chunk 4096]

A step is one flce_fwd_bwd call over one batch: logits GEMM with the
online-logsumexp epilogue, dZ formation, dX and dW GEMMs, loss -- the whole
hot path, with inputs resident in HBM.  Prints ONE JSON line with tokens/s
(value), the roofline of the dominant kernel (per-kernel HIP events recorded
on the call's stream inside the timed region) and the float64 CPU oracle
timed on a bounded token sample of the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused linear-CE fwd+bwd tokens/s and % bf16 MFMA peak, H=4096 V=128256"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA (bf16) / fp32 vector


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", type=int, default=4)
    p.add_argument("--chunk", type=int, default=4096)
    p.add_argument("--cpu-sample", type=int, default=256,
                   help="tokens of the workload the CPU oracle is timed on (0 = skip)")
    p.add_argument("--no-timing", action="store_true",
                   help="time without per-kernel events (no roofline)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (3 times), "
                        "to scale HBM byte counters")
    return p.parse_args()


def calibrate_copy(mib: int):
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "repeats": 3}), flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import linear_cross_entropy_02_amd as flce
    import workloads

    wl = workloads.WORKLOADS[args.workload]
    t_gen = time.time()
    inp = workloads.generate(wl, keep_f32=args.cpu_sample > 0)
    X, W, y = workloads.to_torch(inp, "cuda")
    print(f"[bench] inputs for {wl.name} ready in {time.time() - t_gen:.1f}s", file=sys.stderr,
          flush=True)
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=args.chunk)
    out = op.alloc_outputs(wl.T, "cuda")
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction, out=out)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    timing = not args.no_timing
    if timing:
        flce.flce_timing_enable(op.handle, True)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction, out=out)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    loss = float(out["loss"].item())
    assert np.isfinite(loss), loss

    T, H, V = wl.T, wl.H, wl.V
    flops = 6.0 * T * H * V
    tokens_per_s = T / (ms * 1e-3)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]

    roofline = None
    kernels = {}
    if timing:
        names = flce.flce_timing_kinds()
        for k, name in enumerate(names):
            tot, n = flce.flce_timing_read(op.handle, k)
            if n:
                kernels[name] = {"total_ms": tot / args.steps, "launches_per_step": n / args.steps,
                                 "avg_ms": tot / n}
        flce.flce_timing_enable(op.handle, False)
        dom = max(kernels, key=lambda k: kernels[k]["total_ms"])
        C = op.chunk_tokens
        n_chunks = -(-T // C)
        if dom in ("logits_gemm", "dx_gemm", "dw_gemm"):
            # each GEMM launch contracts one chunk: 2 * C_chunk * H * V flops
            flop_per_launch = 2.0 * T * H * V / n_chunks
            achieved = flop_per_launch / (kernels[dom]["avg_ms"] * 1e-3) / 1e12
            roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                        "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                        "traffic": None}
        else:
            roofline = {"kernel": dom, "bound": "hbm", "achieved": None, "peak": 8000.0,
                        "unit": "GB/s", "frac": None, "traffic": None}

    cpu = None
    if args.cpu_sample > 0:
        from oracle import flce_reference
        ns = min(args.cpu_sample, T)
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        t0 = time.time()
        flce_reference(inp.X[:ns], inp.W, inp.y[:ns], wl.ignore_index, wl.reduction, chunk=256)
        dt = time.time() - t0
        cpu = {"value": round(ns / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"first {ns} of {T} tokens of {wl.name} (full W), float64 numpy oracle, "
                         f"{dt:.1f}s"}

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "T": T, "H": H, "V": V, "chunk_tokens": op.chunk_tokens,
                   "reduction": wl.reduction, "ignore_frac": wl.ignore_frac,
                   "targets": wl.targets},
        "tflops": round(tflops, 1), "mfma_peak_frac": round(tflops / peak, 4),
        "roofline": roofline, "cpu_baseline": cpu, "kernels": kernels,
        "workspace_bytes": op.workspace_bytes,
    }
    op.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
