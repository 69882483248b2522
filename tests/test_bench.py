"""Host logic of bench.py on the CPU: the one-GPU refusal, the per-kernel
roofline arithmetic, the traffic lookup keyed on the kernel sources, and the
kernel names the profile summaries use."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       env={**os.environ, **env}, stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_per_kernel_rooflines():
    T, H, V = 1024, 256, 1000
    kernels = {"logits_gemm": {"total_ms": 2.0}, "dx_gemm": {"total_ms": 1.0},
               "fixup_dz": {"total_ms": 0.5}, "transpose_w": {"total_ms": 0.25},
               "finalize": {"total_ms": 0.125}, "loss": {"total_ms": 0.01}}
    r = bench.per_kernel_rooflines(kernels, T, H, V, "bf16", 2500.0)
    assert set(r) == {"logits_gemm", "dx_gemm", "fixup_dz", "transpose_w", "finalize"}
    flops = 2.0 * T * H * V
    assert r["logits_gemm"]["achieved"] == round(flops / 2e-3 / 1e12, 1)
    assert r["dx_gemm"]["frac"] == round(flops / 1e-3 / 1e12 / 2500.0, 4)
    # the dZ pass: read the exponentials, write dZ^T (bf16)
    assert r["fixup_dz"]["achieved"] == round(2.0 * T * V * 2 / 0.5e-3 / 1e9, 1)
    assert r["transpose_w"]["achieved"] == round(2.0 * V * H * 2 / 0.25e-3 / 1e9, 1)
    # 16 bytes per (token, 128-column tile): ceil(1000 / 128) = 8 tiles
    assert r["finalize"]["achieved"] == round(16.0 * 8 * T / 0.125e-3 / 1e9, 1)
    assert r["finalize"]["bound"] == "hbm" and r["finalize"]["unit"] == "GB/s"
    # dZ written in place as well: one more T x V; fp32 doubles the bytes
    r2 = bench.per_kernel_rooflines(kernels, T, H, V, "f32", 157.3, dz_in_place=True)
    assert r2["fixup_dz"]["achieved"] == round(3.0 * T * V * 4 / 0.5e-3 / 1e9, 1)
    # in place with dW reading dZ as stored: no dZ^T
    r3 = bench.per_kernel_rooflines(kernels, T, H, V, "bf16", 2500.0, dz_in_place=True, dzt=False)
    assert r3["fixup_dz"]["achieved"] == round(2.0 * T * V * 2 / 0.5e-3 / 1e9, 1)


def test_dw_reads_stored_rule():
    assert bench.dw_reads_stored("bf16", 4096, 128256, 2048, 4)        # 2.1 GB of P
    assert not bench.dw_reads_stored("bf16", 4104, 128256, 2048, 4)    # wider than 4096
    assert not bench.dw_reads_stored("f32", 512, 16000, 2048, 1)
    assert bench.dw_reads_stored("bf16", 512, 128256, 8192, 1)        # just under 2^31 bytes
    assert not bench.dw_reads_stored("bf16", 512, 128256, 8192, 2)    # over 2^31 bytes of P


def test_traffic_is_reported_only_for_the_sources_and_launch_it_was_taken_with(tmp_path,
                                                                             monkeypatch):
    rec = {"source_hash": bench.kernel_source_hash(), "launch": [2048, 4, False],
           "kernels": {"gemm<bf16,256x256,4w,LogitsEpi<bf16, false>>":
                       {"read_bytes": 3.0e9, "write_bytes": 0.5e9},
                       "gemm<bf16,256x256,4w,StoreEpi<float, false>>":
                       {"read_bytes": 2.0e9, "write_bytes": 0.25e9},
                       "gemm<bf16,256x256,4w,StoreEpi<float, true>>":
                       {"read_bytes": 9.0e9, "write_bytes": 2.0e9}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(path))
    assert bench.measured_traffic("logits_gemm", (2048, 4, False)) == 3_500_000_000
    assert bench.measured_traffic("dx_gemm", (2048, 4, False)) == 2_250_000_000
    assert bench.measured_traffic("dw_gemm", (2048, 4, False)) == 11_000_000_000
    assert bench.measured_traffic("fixup_dz", (2048, 4, False)) is None
    assert bench.measured_traffic("logits_gemm", (4096, 1, False)) is None   # other launch
    assert bench.measured_traffic("logits_gemm", (2048, 4, True)) is None    # W^T copy
    path.write_text(json.dumps({**rec, "source_hash": "0" * 16}))
    assert bench.measured_traffic("logits_gemm", (2048, 4, False)) is None   # other sources
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("logits_gemm", (2048, 4, False)) is None


def test_committed_traffic_matches_the_current_sources():
    # the committed counter summary is the one the bench line reports: it must
    # have been taken with the kernel sources in the tree
    with open(bench.TRAFFIC_JSON) as f:
        rec = json.load(f)
    assert rec["source_hash"] == bench.kernel_source_hash()


def test_short_kernel_names():
    n = bench.short_kernel_name(
        "void flce::gemm_nt_kernel<flce::bf16, 256, 256, 4, flce::LogitsEpi<flce::bf16, false>, "
        "false>(flce::GemmShape, flce::LogitsEpi<flce::bf16, false>)")
    assert n == "gemm<bf16,256x256,4w,LogitsEpi<bf16, false>>"
    n = bench.short_kernel_name(
        "void flce::gemm_nt_kernel<flce::bf16, 128, 128, 4, flce::StoreEpi<float, false>, "
        "true>(flce::GemmShape, flce::StoreEpi<float, false>)")
    assert n == "gemm<bf16,128x128,4w,StoreEpi<float, false>,Bstored>"
    n = bench.short_kernel_name(
        "void flce::gemm_nt_kernel<flce::bf16, 256, 256, 4, flce::StoreEpi<float, true>, "
        "false, true>(flce::GemmShape, flce::StoreEpi<float, true>)")
    assert n == "gemm<bf16,256x256,4w,StoreEpi<float, true>,Astored>"


def test_the_kernel_hash_follows_the_code_not_the_comments():
    a = 'int f(int x) { // twice x\n  return 2 * x; /* plain */ }\nconst char* s = "a//b";\n'
    b = '/* a header comment */\nint f(int x) {\n    return 2 * x;\n}\nconst char* s = "a//b"; // note\n'
    assert bench.code_tokens(a) == bench.code_tokens(b)
    assert bench.code_tokens(a) != bench.code_tokens(a.replace("2 * x", "3 * x"))
    assert bench.code_tokens(a) != bench.code_tokens(a.replace('"a//b"', '"a// b"'))
    assert bench.code_tokens("char c = '\\''; // x\nint y;") == "char c = '\\''; int y;"
