"""Benchmark: fused linear cross-entropy forward+backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--chunk C] [--dw-chunks G]

A step is one flce_fwd_bwd call over one batch: logits GEMM with the
online-logsumexp epilogue, dZ formation, dX and dW GEMMs, loss -- the whole
hot path, with inputs resident in HBM.  Prints ONE JSON line with tokens/s
(value) from K steps timed with nothing but events between them, the GPU
clock sampled over a few seconds of the same steps run afterwards, the roofline of the dominant kernel
(from a separate pass of a few more steps with a HIP event pair around every
launch on the call's stream) and the float64 CPU oracle timed on a bounded
token sample of the same workload (cpu_baseline).
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
METRIC_FWD = "forward-only per-token log-probs tokens/s and % bf16 MFMA peak, H=4096 V=128256"
METRIC_DISTILL = ("soft-target (distillation) fwd+bwd tokens/s and % bf16 MFMA peak, "
                  "H=4096 V=128256, teacher on the fly")
METRIC_SHARD = ("vocabulary-parallel shard (1 of {n}) fwd+bwd tokens/s and % bf16 MFMA peak, "
                "H=4096 V=128256")
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA peaks, bf16 and fp32
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_JSON = os.path.join(PROFILES, "traffic.json")
KERNEL_SOURCES = ("linear_cross_entropy_02_amd/csrc/gemm.h",
                  "linear_cross_entropy_02_amd/csrc/common.h",
                  "linear_cross_entropy_02_amd/csrc/kernels.hip",
                  "linear_cross_entropy_02_amd/csrc/kernels.h",
                  "linear_cross_entropy_02_amd/csrc/flce_api.cpp")
# rocprofv3 runs whose CSV output --summarize-profiles reads (run from the repo root)
PROFILE_CMDS = {
    "kt": "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_kt -o run -- "
          "python3 bench.py --steps 3 --warmup 1 --cpu-sample 0 --clock-seconds 0 > gpurun_out/prof_kt/bench.json",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof_fetch -o run -- "
             "python3 bench.py --steps 1 --warmup 1 --cpu-sample 0 --no-timing",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof_write -o run -- "
             "python3 bench.py --steps 1 --warmup 1 --cpu-sample 0 --no-timing",
    "cal_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/prof_cal_fetch -o run -- "
                 "python3 bench.py --calibrate-copy 1024",
    "cal_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/prof_cal_write -o run -- "
                 "python3 bench.py --calibrate-copy 1024",
    "mfma": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_LDS_BANK_CONFLICT "
            "SQ_LDS_IDX_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE --output-format csv "
            "-d gpurun_out/prof_mfma -o run -- python3 bench.py --steps 1 --warmup 1 --cpu-sample 0 "
            "--no-timing",
    "mfma_util": "rocprofv3 --pmc MfmaUtil --output-format csv -d gpurun_out/prof_mfma_util -o run -- "
                 "python3 bench.py --steps 1 --warmup 1 --cpu-sample 0 --no-timing",
    "stall1": "rocprofv3 --pmc SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_ANY "
              "SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVES --output-format csv "
              "-d gpurun_out/prof_stall1 -o run -- python3 bench.py --steps 1 --warmup 1 --cpu-sample 0 "
              "--no-timing",
    "stall2": "rocprofv3 --pmc SQ_LDS_CMD_FIFO_FULL SQ_LDS_DATA_FIFO_FULL SQ_LDS_IDX_ACTIVE "
              "SQ_ACTIVE_INST_VMEM SQ_INST_LEVEL_LDS SQ_INST_LEVEL_VMEM SQ_BUSY_CYCLES GRBM_GUI_ACTIVE "
              "--output-format csv -d gpurun_out/prof_stall2 -o run -- python3 bench.py --steps 1 "
              "--warmup 1 --cpu-sample 0 --no-timing",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", type=int, default=4)
    p.add_argument("--chunk", type=int, default=0,
                   help="tokens per chunk (0 = the workload's launch configuration)")
    p.add_argument("--dw-chunks", type=int, default=0,
                   help="token chunks per dW GEMM (the exponentials, or the dZ^T, of that "
                        "many chunks are kept: more than 1 needs (G - 1) C V more workspace; "
                        "0 = the workload's launch configuration)")
    p.add_argument("--weight-copy", choices=("auto", "on", "off"), default="auto",
                   help="dX through a transposed copy of W made per call (on) or reading W "
                        "as stored (off; bf16, no copy in the workspace); auto = the "
                        "workload's launch configuration")
    p.add_argument("--dz-in-place", choices=("auto", "on", "off"), default="auto",
                   help="write dZ over the exponentials and dZ^T for the dX and dW "
                        "contractions (FLCE_FLAG_DZ_IN_PLACE, on) or form it inside them (off); "
                        "auto = the workload's launch configuration")
    p.add_argument("--cpu-sample", type=int, default=3072,
                   help="tokens of the workload the CPU oracle is timed on (0 = skip)")
    p.add_argument("--vocab-shards", type=int, default=1, metavar="N",
                   help="time one device's share of an N-way vocabulary-parallel head: "
                        "flce_vocab_shard_forward + flce_vocab_shard_backward on V/N rows "
                        "(the collectives between them are not part of the step)")
    p.add_argument("--distill-teacher-hidden", type=int, default=0, metavar="HT",
                   help="time flce_distill_fwd_bwd with a teacher head of hidden size HT "
                        "(temperature 2) instead of the hard-label path")
    p.add_argument("--forward-only", action="store_true",
                   help="time flce_forward (per-token log-probs and loss, no gradients)")
    p.add_argument("--no-timing", action="store_true",
                   help="skip the per-kernel pass after the timed steps (no roofline)")
    p.add_argument("--clock-seconds", type=float, default=2.0,
                   help="length of the clock pass after the timed steps (0: none)")
    p.add_argument("--kernel-steps", type=int, default=5,
                   help="steps of the per-kernel pass (HIP events around every launch), run "
                        "after the timed steps; at most --steps")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB (3 times), "
                        "to scale HBM byte counters")
    p.add_argument("--inputs", choices=("random", "pow2", "zero"), default="random",
                   help="operand data: the workload's random X and W (default); the same with "
                        "every bf16 mantissa cleared (sign and exponent kept); or all zero. "
                        "Same work on other bits, to see how the MFMAs' power sets the clock")
    p.add_argument("--mfma-ceiling", action="store_true",
                   help="instead of the benchmark: what the bf16 MFMAs sustain with operands in "
                        "registers (random and zero operands, both instruction shapes, 16 CUs "
                        "and the whole chip), with the clock sampled during each case")
    p.add_argument("--summarize-profiles", metavar="DIR", default=None,
                   help="turn the rocprofv3 CSV output of the PROFILE_CMDS runs under DIR "
                        "into the summaries in profiles/ (no GPU needed)")
    return p.parse_args()


def code_tokens(src: str) -> str:
    """C/C++ source with its comments removed and every run of whitespace
    made one space (comment markers inside string and character literals are
    kept): close to what the compiler sees, so that a comment edit leaves the
    kernels' hash alone."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments and layout ignored)."""
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def short_kernel_name(name: str) -> str:
    import re
    n = name.replace("flce::", "")
    m = re.match(r"void gemm_nt_kernel<([^,]+), (\d+), (\d+), (\d+), (\w+)<([^>]*)>"
                 r"(?:, (true|false))?(?:, (true|false))?", n)
    if m:
        flags = "".join(f",{t}" for t, on in (("Bstored", m.group(7)), ("Astored", m.group(8)))
                        if on == "true")
        return (f"gemm<{m.group(1)},{m.group(2)}x{m.group(3)},{m.group(4)}w,"
                f"{m.group(5)}<{m.group(6).strip()}>{flags}>")
    return n.split("(")[0].replace("void ", "")


def summarize_profiles(d: str):
    """Kernel-time and HBM-traffic summaries from the PROFILE_CMDS outputs."""
    import collections
    import csv

    def rows(sub, fname):
        path = os.path.join(d, sub, fname)
        with open(path) as f:
            return list(csv.DictReader(f))

    stats = rows("prof_kt", "run_kernel_stats.csv")
    lines = ["# Kernel time, fused linear-CE fwd+bwd, llama3-8b head (T=16384, H=4096, V=128256, "
             "bf16, chunk 2048, 4 chunks per dW GEMM)", "",
             "Command (repo root, MI355X):", "", "    " + PROFILE_CMDS["kt"], "",
             "1 warm-up, 3 timed and 3 per-kernel-pass steps (7 calls of flce_fwd_bwd); only the "
             "last 3 carry HIP events around each launch.",
             "", "| kernel | calls | total ms | avg ms | % time |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {short_kernel_name(r['Name'])} | {r['Calls']} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['AverageNs']) / 1e6:.4f} | "
                     f"{float(r['Percentage']):.2f} |")
    # the bench line printed by the same profiled run (its stdout, saved
    # beside the trace) against the traced average of its roofline kernel
    try:
        with open(os.path.join(d, "prof_kt", "bench.json")) as f:
            line = json.loads(f.read().strip().splitlines()[-1])
        rf = line["roofline"]
        tag = {"logits_gemm": "LogitsEpi", "dx_gemm": "StoreEpi<float, false>>",
               "dw_gemm": "StoreEpi<float, true>>"}[rf["kernel"]]
        traced = [r for r in stats if tag in short_kernel_name(r["Name"])]
        avg_all = float(traced[0]["AverageNs"]) * 1e-6
        # the same launches the bench line timed: those of its per-kernel
        # pass, the last ones of the trace
        disp = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                for r in rows("prof_kt", "run_kernel_trace.csv")
                if tag in short_kernel_name(r["Kernel_Name"])]
        n_pass = round(line["kernels"][rf["kernel"]]["launches_per_step"] *
                       min(line["steps"], 3))
        avg = sum(disp[-n_pass:]) / n_pass * 1e-6
        frac = rf["flop_per_launch"] / (avg * 1e-3) / 1e12 / rf["peak"]
        lines += ["", f"Bench line of this run: ms_per_step {line['ms_per_step']}, roofline kernel "
                      f"{rf['kernel']} at {rf['avg_launch_ms']:.4f} ms per launch (HIP events "
                      f"around its last {n_pass} launches), frac {rf['frac']}. The trace's "
                      f"durations of those same {n_pass} launches average {avg:.4f} ms: frac "
                      f"{frac:.4f} ({100 * (rf['frac'] / frac - 1):+.2f} %). Over all "
                      f"{len(disp)} launches, warm-up included, the trace averages "
                      f"{avg_all:.4f} ms."]
    except (OSError, KeyError, IndexError, ValueError):
        pass
    lines += ["", f"Kernel sources hash at measurement: {kernel_source_hash()}"]
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, "kernel_stats_llama3_8b_head.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def per_kernel(sub, counter):
        acc = collections.defaultdict(list)
        for r in rows(sub, "run_counter_collection.csv"):
            if r["Counter_Name"] == counter:
                acc[short_kernel_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    cal_bytes = 1024 * 2 ** 20
    cf = per_kernel("prof_cal_fetch", "FETCH_SIZE")
    cw = per_kernel("prof_cal_write", "WRITE_SIZE")
    copy = [k for k in cf if "copyBuffer" in k or "copy" in k.lower()]
    f_scale = cal_bytes / (cf[copy[0]] * 1024)
    w_scale = cal_bytes / (cw[copy[0]] * 1024)
    fetch = per_kernel("prof_fetch", "FETCH_SIZE")
    write = per_kernel("prof_write", "WRITE_SIZE")
    import workloads
    traffic = {"source_hash": kernel_source_hash(),
               "launch": list(workloads.launch_config(4)) + [workloads.weight_copy(4)],
               "fetch_scale": f_scale, "write_scale": w_scale,
               "kernels": {}}
    lines = ["# HBM traffic per launch, fused linear-CE fwd+bwd, llama3-8b head "
             "(T=16384, H=4096, V=128256, bf16, chunk 2048, 4 chunks per dW GEMM)", "",
             "Commands (repo root, MI355X), one counter pass each:", ""]
    lines += ["    " + PROFILE_CMDS[k] for k in ("fetch", "write", "cal_fetch", "cal_write")]
    lines += ["", f"Calibration: a 1 GiB device-to-device copy reads FETCH_SIZE x {f_scale:.3f} and "
                  f"WRITE_SIZE x {w_scale:.3f} of its true bytes; the figures below are scaled by "
                  "those factors.", "",
              "| kernel | read GB/launch | written GB/launch |", "|---|---|---|"]
    for k in fetch:
        rd = fetch[k] * 1024 * f_scale
        wr = write.get(k, 0.0) * 1024 * w_scale
        traffic["kernels"][k] = {"read_bytes": rd, "write_bytes": wr}
        lines.append(f"| {k} | {rd / 1e9:.3f} | {wr / 1e9:.3f} |")
    calls = {short_kernel_name(r["Name"]): int(r["Calls"]) for r in stats}
    steps_kt = 3 + 1 + 3  # timed, warm-up and per-kernel steps of the "kt" run
    per_step = sum((v["read_bytes"] + v["write_bytes"]) * calls.get(k, 0) / steps_kt
                   for k, v in traffic["kernels"].items() if not k.startswith("__amd"))
    traffic["per_step_bytes"] = per_step
    lines += ["", f"Per fwd+bwd step (launches per step from the kernel trace): "
                  f"{per_step / 1e9:.1f} GB, against {3.42:.2f} GB of algorithmic bytes "
                  "(X, W, targets, dX, fp32 dW, lse)."]
    lines += ["", f"Kernel sources hash at measurement: {traffic['source_hash']}"]
    with open(os.path.join(PROFILES, "hbm_traffic_llama3_8b_head.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(traffic, f, indent=1)
    print("\n".join(lines))

    # MFMA busy and LDS bank conflicts (both counter passes are optional)
    def per_kernel(sub):
        acc = collections.defaultdict(lambda: collections.defaultdict(float))
        n = collections.defaultdict(lambda: collections.defaultdict(int))
        for r in rows(sub, "run_counter_collection.csv"):
            k = short_kernel_name(r["Kernel_Name"])
            acc[k][r["Counter_Name"]] += float(r["Counter_Value"])
            n[k][r["Counter_Name"]] += 1
        return {k: {c: acc[k][c] / n[k][c] for c in acc[k]} for k in acc}
    try:
        raw = per_kernel("prof_mfma")
    except OSError:
        return
    try:
        util = per_kernel("prof_mfma_util")
    except OSError:
        util = {}
    lines = ["# MFMA busy and LDS bank conflicts per launch, fused linear-CE fwd+bwd, llama3-8b "
             "head (T=16384, H=4096, V=128256, bf16, chunk 2048, 4 chunks per dW GEMM)", "",
             "Commands (repo root, MI355X), one counter pass each:", "",
             "    " + PROFILE_CMDS["mfma"], "    " + PROFILE_CMDS["mfma_util"], "",
             "MfmaUtil is rocprofv3's derived metric (percent of the MFMA units' cycles busy over "
             "the launch); bf16 FLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; bank conflicts are "
             "SQ_LDS_BANK_CONFLICT cycles against SQ_LDS_IDX_ACTIVE cycles.", "",
             "| kernel | MfmaUtil % | bf16 TFLOP counted | LDS bank-conflict cycles | "
             "LDS active cycles | conflict % |", "|---|---|---|---|---|---|"]
    for k, c in sorted(raw.items(), key=lambda kv: -kv[1].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0)):
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        if mops <= 0:
            continue
        bc, act = c.get("SQ_LDS_BANK_CONFLICT", 0.0), c.get("SQ_LDS_IDX_ACTIVE", 0.0)
        mu = util.get(k, {}).get("MfmaUtil")
        lines.append(f"| {k} | {mu:.1f} | {mops * 512 / 1e12:.3f} | {bc:.3e} | {act:.3e} | "
                     f"{100.0 * bc / act if act else 0.0:.2f} |" if mu is not None else
                     f"| {k} | n/a | {mops * 512 / 1e12:.3f} | {bc:.3e} | {act:.3e} | "
                     f"{100.0 * bc / act if act else 0.0:.2f} |")
    lines += ["", f"Kernel sources hash at measurement: {kernel_source_hash()}"]
    with open(os.path.join(PROFILES, "mfma_lds_counters_llama3_8b_head.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # wait and FIFO counters of the GEMMs (both passes optional)
    try:
        s1, s2 = per_kernel("prof_stall1"), per_kernel("prof_stall2")
    except OSError:
        return
    times = {short_kernel_name(r["Name"]): float(r["AverageNs"]) * 1e-9 for r in stats}
    lines = ["# GEMM stall counters per launch, fused linear-CE fwd+bwd, llama3-8b head (T=16384, "
             "H=4096, V=128256, bf16, chunk 2048, 4 chunks per dW GEMM)", "",
             "Commands (repo root, MI355X), one counter pass each:", "",
             "    " + PROFILE_CMDS["stall1"], "    " + PROFILE_CMDS["stall2"], "",
             "Cycles per launch = GRBM_GUI_ACTIVE / 8 XCDs; SIMD-cycles = that x 1024 SIMDs (one "
             "wave per SIMD). MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMD-cycles; the SQ_WAIT_* "
             "counters count quad-cycles (x 4). Clock = cycles / the launch time of the kernel-time "
             "summary.", "",
             "| kernel | cycles / launch | clock GHz | MFMA busy | waiting on waitcnt / barrier | "
             "waiting for LDS issue | LDS command FIFO full cycles | LDS data FIFO full cycles |",
             "|---|---|---|---|---|---|---|---|"]
    for k, a in sorted(s1.items(), key=lambda kv: -kv[1].get("SQ_VALU_MFMA_BUSY_CYCLES", 0)):
        b = s2.get(k, {})
        if a.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) <= 0 or not b.get("GRBM_GUI_ACTIVE"):
            continue
        cyc = b["GRBM_GUI_ACTIVE"] / 8
        simd = cyc * 1024
        clk = f"{cyc / times[k] / 1e9:.2f}" if times.get(k) else "n/a"
        lines.append(f"| {k} | {cyc:.3e} | {clk} | {100 * a['SQ_VALU_MFMA_BUSY_CYCLES'] / simd:.1f} % | "
                     f"{100 * 4 * a['SQ_WAIT_ANY'] / simd:.1f} % | "
                     f"{100 * 4 * a['SQ_WAIT_INST_LDS'] / simd:.1f} % | "
                     f"{b.get('SQ_LDS_CMD_FIFO_FULL', 0):.2e} | {b.get('SQ_LDS_DATA_FIFO_FULL', 0):.0f} |")
    lines += ["", f"Kernel sources hash at measurement: {kernel_source_hash()}"]
    with open(os.path.join(PROFILES, "gemm_stall_counters_llama3_8b_head.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def measured_traffic(kernel_kind: str, launch):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when the kernel sources or the launch configuration
    (chunk, chunks per dW GEMM, W^T copy) differ from those it was taken
    with."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("source_hash") != kernel_source_hash() or t.get("launch") != list(launch):
        return None
    # logits: LogitsEpi; dX: fp32 split-K partials, else a direct store of the
    # input dtype; dW: the accumulating fp32 store
    tags = {"logits_gemm": ("LogitsEpi",), "dx_gemm": ("StoreEpi<float, false>", "StoreEpi<bf16, false>"),
            "dw_gemm": ("StoreEpi<float, true>",)}.get(kernel_kind, ())
    for tag in tags:
        for k, v in t["kernels"].items():
            if tag in k:
                return round(v["read_bytes"] + v["write_bytes"])
    return None


def dw_reads_stored(dtype, H, V, chunk, dw_chunks) -> bool:
    """Whether the dW contraction reads P (exponentials or dZ) as stored,
    with no dZ^T written: the rule include/flce.h states (bf16, H <= 4096,
    the G chunks of P under 2^31 bytes)."""
    vpad = -(-V // 256) * 256
    return dtype == "bf16" and H <= 4096 and dw_chunks * chunk * vpad * 2 < 2 ** 31


def per_kernel_rooflines(kernels, T, H, V, dtype, mfma_peak, dz_in_place=False, dzt=True):
    """Achieved rate of each timed kernel of one fwd+bwd step against its own
    bound, from algorithmic work only: 2 T H V flops for each contraction;
    for the bandwidth passes the bytes they must move (the dZ pass reads the
    exponentials and writes dZ over them with dz_in_place and dZ^T with
    dzt; its rewrite of the few tiles whose reference lies below their
    row's is not counted; a transpose reads and writes its matrix once; the
    merge reads the (max, sum, argmax) partials and writes alpha, 16 bytes
    per (token, 128-column tile))."""
    es = 2 if dtype == "bf16" else 4
    nt = -(-V // 128)
    fixup_bytes = (1.0 + float(dz_in_place) + float(dzt)) * T * V * es
    work = {"logits_gemm": ("mfma", 2.0 * T * H * V), "dx_gemm": ("mfma", 2.0 * T * H * V),
            "dw_gemm": ("mfma", 2.0 * T * H * V), "fixup_dz": ("hbm", fixup_bytes),
            "transpose_w": ("hbm", 2.0 * V * H * es), "transpose_x": ("hbm", 2.0 * T * H * es),
            "finalize": ("hbm", 16.0 * nt * T)}
    out = {}
    for name, (bound, per_step) in work.items():
        k = kernels.get(name)
        if not k or not k["total_ms"]:
            continue
        rate = per_step / (k["total_ms"] * 1e-3)
        if bound == "mfma":
            out[name] = {"bound": "mfma", "achieved": round(rate / 1e12, 1), "unit": "TFLOP/s",
                         "frac": round(rate / 1e12 / mfma_peak, 4)}
        else:
            out[name] = {"bound": "hbm", "achieved": round(rate / 1e9, 1), "unit": "GB/s",
                         "frac": round(rate / 1e9 / 8000.0, 4)}
    return out


class ClockSampler:
    """GFX clock and socket power of device 0 sampled every 20 ms from a side
    thread (amdsmi GPU metrics) while steps run.  The firmware
    refreshes that table more slowly than it is read, and its first values
    can predate the load, so the summary is the median (and range) of the
    samples taken in the second half of the window; None without amdsmi."""

    def __init__(self, period_s: float = 0.02):
        import threading
        self.period_s = period_s
        self.samples = []          # (seconds since start, MHz, watts or None)
        self._halt = threading.Event()
        self._thread = None
        self._handle = None
        self._error = None
        self._t0 = 0.0

    def _read(self):
        import amdsmi
        m = amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = m.get("current_gfxclks")
        clks = [c for c in clks if isinstance(c, (int, float)) and 0 < c < 10000] \
            if isinstance(clks, (list, tuple)) else []
        if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
            clks = [m["current_gfxclk"]]
        p = m.get("current_socket_power")
        p = float(p) if isinstance(p, (int, float)) and 0 < p < 5000 else None
        if clks:
            self.samples.append((time.time() - self._t0, sum(clks) / len(clks), p))

    def _run(self):
        while not self._halt.wait(self.period_s):
            try:
                self._read()
            except Exception as e:  # metrics unavailable on this machine
                self._error = repr(e)
                return

    def start(self):
        import threading
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._handle = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:
            self._error = repr(e)
            self._handle = None
            return
        self._t0 = time.time()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        span = time.time() - self._t0
        if self._thread is not None:
            self._halt.set()
            self._thread.join()
        try:
            if self._handle is not None:
                import amdsmi
                amdsmi.amdsmi_shut_down()
        except Exception:
            pass
        late = [s for s in self.samples if s[0] >= 0.5 * span]
        if not late:
            return {"gfx_clock_mhz": None, "error": self._error}
        clk = sorted(s[1] for s in late)
        pw = sorted(s[2] for s in late if s[2] is not None)
        out = {"gfx_clock_mhz": clk[len(clk) // 2], "gfx_clock_mhz_min": clk[0],
               "gfx_clock_mhz_max": clk[-1], "samples": len(clk),
               "window_s": round(span / 2, 3), "nominal_peak_clock_mhz": 2400,
               "source": "amdsmi gpu metrics current_gfxclks (mean of the XCDs), median of the "
                         "samples in the second half of a window of back-to-back steps"}
        if pw:
            out["socket_power_w"] = pw[len(pw) // 2]
        return out


def blas_threads():
    """Threads of the BLAS numpy uses (threadpoolctl), or None."""
    try:
        import numpy  # noqa: F401  (loads the BLAS the pool query reports)
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        return {"library": info[0].get("internal_api"), "threads": info[0].get("num_threads")} \
            if info else None
    except Exception:
        return None


def calibrate_copy(mib: int):
    import torch
    n = mib * 2 ** 20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n * 4, "repeats": 3}), flush=True)


def mfma_ceiling():
    """Rates of the MFMA probe (libflce_probe.so): for each instruction shape,
    operand kind and grid, one calibration launch, then launches sized to
    about 0.25 s each, timed with an event pair on the current stream; the
    reported rate is the median of 4 such launches after one warm-up, with
    the clock sampled over them.  One JSON line."""
    import torch

    from linear_cross_entropy_02_amd import probe

    peak = PEAK_TFLOPS["bf16"]
    stream = torch.cuda.current_stream()
    sink = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
    results = []

    def timed(shape, blocks, iters, rnd):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        probe.mfma_stream(shape, blocks, iters, rnd, sink, stream)
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b)

    for blocks in (16, 256, 512):
        for shape in (16, 32):
            for rnd in (True, False):
                ms0 = timed(shape, blocks, 2000, rnd)
                iters = max(2000, int(2000 * 250.0 / max(ms0, 1e-3)))
                timed(shape, blocks, iters, rnd)
                sampler = ClockSampler()
                sampler.start()
                times = sorted(timed(shape, blocks, iters, rnd) for _ in range(4))
                clock = sampler.stop()
                ms = 0.5 * (times[1] + times[2])
                zero_ok = rnd or bool((sink[:blocks * 256] == 0).all().item())
                tf = probe.mfma_flops(shape, blocks, iters) / (ms * 1e-3) / 1e12
                # a CU's share of the peak: 16 CUs can reach 16/256 of it
                share = peak * min(blocks, 256) / 256.0
                r = {"instruction": ("v_mfma_f32_16x16x32_bf16" if shape == 16 else
                                     "v_mfma_f32_32x32x16_bf16"),
                     "operands": "random" if rnd else "zero", "blocks": blocks,
                     "waves_per_simd": max(1, blocks // 256), "iters": iters,
                     "ms_per_launch": round(ms, 3), "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / peak, 4),
                     "frac_of_cu_share": round(tf / share, 4),
                     "gfx_clock_mhz": clock.get("gfx_clock_mhz"),
                     "socket_power_w": clock.get("socket_power_w"),
                     "zero_sink_ok": zero_ok}
                results.append(r)
                print(f"[mfma-ceiling] {r['instruction']} {r['operands']} blocks={blocks}: "
                      f"{r['tflops']} TF/s ({100 * r['frac_of_peak']:.1f} % of peak), "
                      f"clock {r['gfx_clock_mhz']} MHz", file=sys.stderr, flush=True)
    print(json.dumps({"mfma_ceiling": results, "peak_tflops": peak,
                      "device": torch.cuda.get_device_name(0)}), flush=True)


def main():
    args = parse()
    if args.mfma_ceiling:
        mfma_ceiling()
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
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
    mode = ("forward" if args.forward_only else "shard" if args.vocab_shards > 1 else
            "distill" if args.distill_teacher_hidden > 0 else "fwd_bwd")
    chunk, dwc = workloads.launch_config(args.workload, mode)
    args.chunk = args.chunk or chunk
    args.dw_chunks = args.dw_chunks or dwc
    wcopy = (workloads.weight_copy(args.workload, mode) if args.weight_copy == "auto"
             else args.weight_copy == "on")
    args.dz_in_place = (workloads.dz_in_place(args.workload, mode) if args.dz_in_place == "auto"
                        else args.dz_in_place == "on")
    t_gen = time.time()
    inp = workloads.generate(wl, keep_f32=args.cpu_sample > 0)
    X, W, y = workloads.to_torch(inp, "cuda")
    if args.inputs != "random":
        for t in (X, W):
            if args.inputs == "zero":
                t.zero_()
            elif t.dtype == torch.bfloat16:
                t.view(torch.int16).bitwise_and_(-128)    # 0xFF80: sign and exponent
            else:
                t.view(torch.int32).bitwise_and_(-8388608)  # 0xFF800000
        args.cpu_sample = 0  # the oracle leg times the random inputs only
    print(f"[bench] inputs for {wl.name} ready in {time.time() - t_gen:.1f}s", file=sys.stderr,
          flush=True)
    n_shards = max(1, args.vocab_shards)
    fwd_only = args.forward_only
    Ht = args.distill_teacher_hidden
    if Ht > 0:
        tinp = workloads.generate(wl.with_shape(H=Ht, seed=wl.seed + 500))
        Xq, Wq, _ = workloads.to_torch(tinp, "cuda")
        del tinp
        op = flce.FusedDistillationCrossEntropy(wl.H, wl.V, Ht, wl.dtype, chunk_tokens=args.chunk,
                                                dw_chunks=args.dw_chunks, weight_copy=wcopy)
        out = op.distill(X, W, Xq, Wq, y, 2.0, wl.ignore_index, wl.reduction)

        def step():
            op.distill(X, W, Xq, Wq, y, 2.0, wl.ignore_index, wl.reduction, out=out)
    elif n_shards > 1:
        # the whole vocabulary's lse, as the collectives after step 1 would give it
        full = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=args.chunk)
        lse_g = full.forward(X, W, y, wl.ignore_index, wl.reduction)["lse"]
        full.close()
        Vs = wl.V // n_shards
        Ws = W[:Vs].contiguous()
        op = flce.FusedLinearCrossEntropy(wl.H, Vs, wl.dtype, chunk_tokens=args.chunk,
                                          dw_chunks=args.dw_chunks, weight_copy=wcopy)
        red = flce.FLCE_MEAN if wl.reduction == "mean" else flce.FLCE_SUM
        parts = [torch.empty(wl.T, device="cuda") for _ in range(3)]
        amax = torch.empty(wl.T, dtype=torch.int32, device="cuda")
        dXp = torch.empty(wl.T, wl.H, dtype=X.dtype, device="cuda")
        dWs = torch.empty(Vs, wl.H, dtype=torch.float32, device="cuda")
        out = {"loss": lse_g[:1]}

        def step():
            st1 = flce.flce_vocab_shard_forward(op.handle, X, Ws, y, wl.T, wl.ignore_index, 0,
                                                wl.V, parts[0], parts[1], amax, parts[2])
            st2 = flce.flce_vocab_shard_backward(op.handle, X, Ws, y, wl.T, wl.ignore_index, 0,
                                                 wl.V, red, lse_g, dXp, dWs)
            assert st1 == flce.FLCE_OK and st2 == flce.FLCE_OK, (st1, st2)
    else:
        # the forward-only call runs on a forward-only handle (no backward buffers)
        op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=args.chunk,
                                          dw_chunks=args.dw_chunks, weight_copy=wcopy,
                                          dz_in_place=args.dz_in_place, forward_only=fwd_only)
    if n_shards > 1 or Ht > 0:
        pass  # step() is set above
    elif fwd_only:
        out = op.forward(X, W, y, wl.ignore_index, wl.reduction)

        def step():
            op.forward(X, W, y, wl.ignore_index, wl.reduction, out=out)
    else:
        out = op.alloc_outputs(wl.T, "cuda")

        def step():
            op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction, out=out)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # Timed region: the K steps alone, no per-kernel instrumentation.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info()[0]
    start.record(stream)
    marks[0].record(stream)
    for i in range(args.steps):
        step()
        marks[i + 1].record(stream)
    stop.record(stream)
    torch.cuda.synchronize()
    free_after = torch.cuda.mem_get_info()[0]
    ms = start.elapsed_time(stop) / args.steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    loss = float(out["loss"].item())
    assert np.isfinite(loss), loss
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)

    # Clock pass, after and apart from the timed region: the same step run
    # back to back for a few seconds while the clock is sampled (the metrics
    # table refreshes too slowly to be read over the short timed region).
    clock = None
    if args.clock_seconds > 0 and not args.no_timing:
        sampler = ClockSampler()
        sampler.start()
        t_end = time.time() + args.clock_seconds
        n_clock = 0
        while time.time() < t_end:
            for _ in range(4):
                step()
            n_clock += 4
            torch.cuda.synchronize()
        clock = sampler.stop()
        clock["steps"] = n_clock

    T, H, V = wl.T, wl.H, wl.V
    # fwd+bwd: three contractions of 2 T H V flops; forward only: the logits;
    # a vocabulary shard: its logits twice (step 1 and the recompute in
    # step 2) and its dX and dW contributions, over V / N columns
    if n_shards > 1:
        V = V // n_shards
    flops = (8.0 if n_shards > 1 else 2.0 if fwd_only else 6.0) * T * H * V
    if Ht > 0:  # the teacher's logits on top of the student's three contractions
        flops = 6.0 * T * H * V + 2.0 * T * Ht * V
    tokens_per_s = T / (ms * 1e-3)
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]

    # Per-kernel pass, after and apart from the timed region: the same steps
    # again with a HIP event pair recorded on the call's stream around every
    # launch; the roofline of the dominant kernel comes from these durations.
    roofline = None
    kernels = {}
    kernel_rooflines = None
    ksteps = 0 if args.no_timing else max(1, min(args.steps, args.kernel_steps))
    if ksteps:
        flce.flce_timing_enable(op.handle, True)
        for _ in range(ksteps):
            step()
        torch.cuda.synchronize()
        names = flce.flce_timing_kinds()
        for k, name in enumerate(names):
            tot, n = flce.flce_timing_read(op.handle, k)
            if n:
                kernels[name] = {"total_ms": tot / ksteps, "launches_per_step": n / ksteps,
                                 "avg_ms": tot / n}
        flce.flce_timing_enable(op.handle, False)
        source = (f"HIP event pair around each launch on the call's stream, {ksteps} steps "
                  "after the timed region")
        dom = max(kernels, key=lambda k: kernels[k]["total_ms"])
        if dom in ("logits_gemm", "dx_gemm", "dw_gemm"):
            # each of the contractions does 2 T H V flops per step, split over
            # its launches (one per chunk; one per dW group for dW); a
            # vocabulary shard runs its logits GEMM twice per step
            nrep = 2.0 if (n_shards > 1 and dom == "logits_gemm") else 1.0
            if Ht > 0 and dom == "logits_gemm":  # student and teacher logits
                nrep = (H + Ht) / H
            flop_per_launch = nrep * 2.0 * T * H * V / kernels[dom]["launches_per_step"]
            achieved = flop_per_launch / (kernels[dom]["avg_ms"] * 1e-3) / 1e12
            roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
                        "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                        "traffic": None if (fwd_only or n_shards > 1 or Ht > 0 or
                                            args.workload != 4) else
                        measured_traffic(dom, (op.chunk_tokens, op.dw_chunks, wcopy)),
                        "flop_per_launch": flop_per_launch,
                        "avg_launch_ms": round(kernels[dom]["avg_ms"], 5), "source": source}
        else:
            roofline = {"kernel": dom, "bound": "hbm", "achieved": None, "peak": 8000.0,
                        "unit": "GB/s", "frac": None, "traffic": None, "source": source}
        if not (fwd_only or n_shards > 1 or Ht > 0):
            kernel_rooflines = per_kernel_rooflines(
                kernels, T, H, V, wl.dtype, peak, args.dz_in_place,
                not dw_reads_stored(wl.dtype, H, V, op.chunk_tokens, op.dw_chunks))

    cpu = None
    if args.cpu_sample > 0 and n_shards == 1 and Ht == 0:
        from oracle import flce_reference
        ns = min(args.cpu_sample, T)
        blas = blas_threads()
        threads = (blas or {}).get("threads") or len(os.sched_getaffinity(0))
        t0 = time.time()
        flce_reference(inp.X[:ns], inp.W, inp.y[:ns], wl.ignore_index, wl.reduction, chunk=256,
                       want_grads=not fwd_only)
        dt = time.time() - t0
        cpu = {"value": round(ns / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "blas": blas, "host_cpus": len(os.sched_getaffinity(0)),
               "sample": f"first {ns} of {T} tokens of {wl.name} (full W), float64 numpy oracle, "
                         f"{dt:.1f}s"}

    line = {
        "metric": (METRIC_DISTILL if Ht > 0 else METRIC_SHARD.format(n=n_shards) if n_shards > 1 else
                   METRIC_FWD if fwd_only else METRIC), "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic" if args.inputs == "random" else f"synthetic ({args.inputs} X, W)",
        "config": {"workload": wl.name, "T": T, "H": H, "V": V, "chunk_tokens": op.chunk_tokens,
                   "dw_chunks": op.dw_chunks, "weight_copy": wcopy, "dz_in_place": args.dz_in_place,
                   "vocab_shards": n_shards,
                   "V_total": wl.V,
                   "teacher_hidden": Ht,
                   "reduction": wl.reduction, "ignore_frac": wl.ignore_frac,
                   "targets": wl.targets},
        "tflops": round(tflops, 1), "mfma_peak_frac": round(tflops / peak, 4),
        "roofline": roofline, "cpu_baseline": cpu, "clock": clock, "kernels": kernels,
        "kernel_rooflines": kernel_rooflines,
        "ms_per_step_median": round(ms_median, 3),
        "workspace_bytes": op.workspace_bytes,
        # the no-T x V-buffer check: workspace against a bf16 T x V buffer,
        # and device memory taken during the timed calls (none is allocated)
        "workspace_vs_TxV_bf16": round(op.workspace_bytes / (2.0 * T * V), 4),
        "device_alloc_in_calls_bytes": max(0, free_before - free_after),
    }
    op.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
