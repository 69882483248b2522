"""The GEMM kernels' hand-kept wait states, checked on their gfx950 assembly
(CPU only: hipcc cross-compiles).

The MFMAs are inline asm, which the compiler's hazard recognizer does not
look inside, so the distances the hardware needs are kept by the code:
  * two wait states between a VALU write of a VGPR and an MFMA reading it
    as a source (any register copy the compiler places before an asm MFMA);
  * a drain between the last MFMA of a K loop and the first non-MFMA read of
    its accumulators (s_nop 7 three times in the last iteration and four
    times after the loop; the check asks for 18, what a 16-pass MFMA result
    needs, and finds at least 30 in every kernel).
isa_hazards.check scans every gemm_nt_kernel instantiation straight through
its branches; a planted hazard shows that it catches each kind.
"""
import os
import subprocess

import pytest

import isa_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    from linear_cross_entropy_02_amd import build as b
    try:
        cc = b.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("isa") / "kernels.s")
    flags = [f for f in b.HIPCC_FLAGS if f != "-fPIC"]
    r = subprocess.run([cc, "-x", "hip", "--cuda-device-only", "-S",
                        os.path.join(b.CSRC, "kernels.hip"), "-o", out] + flags,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    return open(out).read()


def test_gemm_kernels_keep_their_wait_states(device_asm):
    kernels = {f for f, _, _ in isa_hazards.instructions(device_asm)
               if f and "gemm_nt_kernel" in f}
    assert len(kernels) >= 20, sorted(kernels)
    n_mfma = sum(1 for f, opc, _ in isa_hazards.instructions(device_asm)
                 if f in kernels and opc.startswith("v_mfma"))
    assert n_mfma > 1000
    problems = isa_hazards.check(device_asm, lambda n: "gemm_nt_kernel" in n)
    assert not problems, "\n".join(problems[:20])


def test_the_check_catches_planted_hazards():
    asm = "\n".join([
        "k:",
        "\tv_mov_b32 v5, v6",                                                # source just written
        "\tv_mfma_f32_16x16x32_bf16 a[0:3], v[2:5], v[8:11], a[0:3]",
        "\ts_nop 7",
        "\tv_accvgpr_read_b32 v7, a1",                                      # 9 wait states later
        "\ts_nop 1",
        "\tv_mfma_f32_16x16x32_bf16 a[4:7], v[12:15], v[8:11], a[4:7]",   # 2 after a VALU: fine
        "\ts_endpgm",
    ])
    problems = isa_hazards.check(asm)
    assert len(problems) == 2, problems
    assert "VALU write" in problems[0] and "v_accvgpr_read_b32" in problems[1]
