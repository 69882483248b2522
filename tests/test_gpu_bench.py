"""bench.py end to end on the GPU: the one JSON line it prints keeps its
contract (metric, throughput, roofline of the dominant kernel, the oracle's
CPU baseline, the clock), on the small 4096 x 512 x 16000 layer and on a few
steps of the default head."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench_line(*argv, timeout=300):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py")] + list(argv)
    print("[gpu-bench]", " ".join(cmd[2:]), flush=True)
    r = subprocess.run(cmd, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       timeout=timeout)
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def check_contract(line, steps, warmup):
    assert line["n_gpus"] == 1 and line["steps"] == steps and line["warmup"] == warmup
    assert line["unit"] == "tokens/s" and line["higher_is_better"] is True
    assert line["scaling"] == "weak" and line["data"] == "synthetic"
    assert line["value"] > 0 and line["ms_per_step"] > 0
    # value = T / step time; ms_per_step is printed to 3 decimals
    T, ms = line["config"]["T"], line["ms_per_step"]
    assert T / ((ms + 5e-4) * 1e-3) - 1 <= line["value"] <= T / ((ms - 5e-4) * 1e-3) + 1
    assert line["device_alloc_in_calls_bytes"] == 0
    rf = line["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 2500.0
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["kernel"] in ("logits_gemm", "dx_gemm", "dw_gemm")
    assert abs(rf["achieved"] - rf["flop_per_launch"] / (rf["avg_launch_ms"] * 1e-3) / 1e12) \
        <= 1e-3 * rf["achieved"] + 0.1
    return rf


def test_bench_line_small_layer():
    line = bench_line("--workload", "2", "--steps", "4", "--warmup", "1", "--kernel-steps", "2",
                      "--clock-seconds", "0.5", "--cpu-sample", "64")
    check_contract(line, 4, 1)
    c = line["config"]
    assert c["workload"] == "layer-B4S1024-H512-V16000" and (c["T"], c["H"], c["V"]) == (4096, 512, 16000)
    assert line["roofline"]["traffic"] is None           # counters are kept for the head only
    cpu = line["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["unit"] == "tokens/s" and cpu["value"] > 0
    assert cpu["cores"] >= 1 and "64 of 4096" in cpu["sample"]
    assert line["workspace_vs_TxV_bf16"] < 1.0


def test_bench_line_default_head():
    line = bench_line("--steps", "2", "--warmup", "1", "--kernel-steps", "1",
                      "--clock-seconds", "0", "--cpu-sample", "0")
    rf = check_contract(line, 2, 1)
    c = line["config"]
    assert c["workload"] == "llama3-8b-head-T16384-H4096-V128256"
    assert (c["T"], c["H"], c["V"]) == (16384, 4096, 128256)
    assert line["cpu_baseline"] is None                  # --cpu-sample 0
    # the committed counter summary matches these sources and this launch
    assert rf["traffic"] is not None and rf["traffic"] > 0
    assert line["workspace_vs_TxV_bf16"] < 1.0
    # every GEMM of the step appears in the per-kernel pass
    for k in ("logits_gemm", "dx_gemm", "dw_gemm", "finalize"):
        assert line["kernels"][k]["total_ms"] > 0, k
