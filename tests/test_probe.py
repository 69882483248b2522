"""The MFMA throughput probe library (libflce_probe.so), on the CPU: its
exports, its work count, the arguments it refuses before touching a device,
and the wait states its asm MFMAs keep in the gfx950 assembly."""
import ctypes
import os
import subprocess

import pytest

import isa_hazards
from linear_cross_entropy_02_amd import probe

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "flce_probe.h")


def lib():
    if not os.path.exists(probe.PROBE_PATH):
        pytest.skip("libflce_probe.so not built")
    return probe.load()


def test_exports_match_header():
    import re
    l = lib()
    declared = set(re.findall(r"\b(flce_probe_\w+)\s*\(", open(HEADER).read()))
    assert declared == set(probe.EXPORTED)
    for name in declared:
        assert getattr(l, name) is not None


def test_flop_count():
    # 4 waves x (16 issues of 16x16x32 or 8 of 32x32x16) per round, 2 flops per FMA
    assert probe.mfma_flops(16, 3, 5) == 4 * 3 * 5 * 16 * (2 * 16 * 16 * 32)
    assert probe.mfma_flops(32, 3, 5) == 4 * 3 * 5 * 8 * (2 * 32 * 32 * 16)
    assert probe.mfma_flops(8, 3, 5) == 0.0


@pytest.mark.parametrize("shape,blocks,iters,sink", [
    (8, 1, 1, 1), (16, 0, 1, 1), (32, 1, 0, 1), (16, 1, 1, 0), (32, -4, 1, 1)])
def test_bad_arguments_refused_before_launch(shape, blocks, iters, sink):
    l = lib()
    ptr = ctypes.c_void_p(0x1000 if sink else 0)
    assert l.flce_probe_mfma_stream(shape, blocks, iters, 1, ptr, None) == 1


def test_probe_kernels_keep_their_wait_states(tmp_path):
    from linear_cross_entropy_02_amd import build as b
    try:
        cc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = str(tmp_path / "probe.s")
    flags = [f for f in b.HIPCC_FLAGS if f != "-fPIC"]
    r = subprocess.run([cc, "-x", "hip", "--cuda-device-only", "-S",
                        os.path.join(b.CSRC, "probe_mfma.hip"), "-o", out] + flags,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    asm = open(out).read()
    kernels = {f for f, _, _ in isa_hazards.instructions(asm) if f and "stream_kernel" in f}
    assert len(kernels) == 2, kernels
    ops = {opc for f, opc, _ in isa_hazards.instructions(asm) if f in kernels}
    assert {"v_mfma_f32_16x16x32_bf16", "v_mfma_f32_32x32x16_bf16"} <= ops
    problems = isa_hazards.check(asm, lambda n: "stream_kernel" in n)
    assert not problems, "\n".join(problems[:20])
