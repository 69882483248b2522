"""Build libflce.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m linear_cross_entropy_02_amd.build

compiles every source under csrc/ on every call (the CPU-only container
cross-compiles gfx950 code objects) and writes the shared library next to
this file, together with libflce_probe.so (the MFMA throughput probe, a
measuring aid that the fused path does not use).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libflce.so")
PROBE_LIB = os.path.join(PKG, "libflce_probe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off (hipcc would emit v_pk_*_f32 by itself)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-result",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out)


# Host-side sanitizer build (the ABI tests run against it on the CPU): every
# -fsanitize applies to the host pass only, the device code is unchanged.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-O1"]


def asan_runtime() -> str:
    """The AddressSanitizer runtime of hipcc's clang (preloaded by a process
    that loads the sanitizer build, since a shared library does not carry it)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    r = subprocess.run([clang, "--print-file-name=libclang_rt.asan-x86_64.so"],
                       stdout=subprocess.PIPE, text=True)
    return r.stdout.strip()


def build(verbose: bool = False, sanitize: bool = False, out: str = LIB,
          defines: tuple = ()) -> str:
    """Compile csrc/ into `out`.  `defines` ("NAME=VALUE") override the
    tuning constants the sources leave open to the build (the logits and dW
    grids' tile-group sizes)."""
    cc = hipcc()
    objdir = os.path.join(PKG, "_build_san" if sanitize else "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src, lang in (("kernels.hip", "hip"), ("flce_api.cpp", "hip")):
        obj = os.path.join(objdir, src.rsplit(".", 1)[0] + ".o")
        cmd = [cc, "-x", lang, "-c", os.path.join(CSRC, src), "-o", obj] + HIPCC_FLAGS
        cmd += [f"-D{d}" for d in defines]
        if sanitize:
            cmd += SANITIZE_FLAGS
        if verbose:
            print(" ".join(cmd))
        _run(cmd)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if sanitize:
        cmd += ["-fsanitize=address,undefined", "-shared-libsan"]
    if verbose:
        print(" ".join(cmd))
    _run(cmd)
    os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False, out: str = PROBE_LIB) -> str:
    """Compile csrc/probe_mfma.hip into its own library `out`."""
    cc = hipcc()
    tmp = out + ".tmp"
    cmd = [cc, "-x", "hip", os.path.join(CSRC, "probe_mfma.hip"), "-shared", "-o", tmp] + HIPCC_FLAGS
    if verbose:
        print(" ".join(cmd))
    _run(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    # python -m linear_cross_entropy_02_amd.build [-v] [-DNAME=VALUE ...]
    print(build(verbose="-v" in sys.argv,
                defines=tuple(a[2:] for a in sys.argv[1:] if a.startswith("-D"))))
    print(build_probe(verbose="-v" in sys.argv))
