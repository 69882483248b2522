"""Binding of libflce_probe.so (include/flce_probe.h): the MFMA throughput
probe that measures what the bf16 matrix instructions sustain with operands
in registers, random or zero.  A measuring aid beside the fused path."""
from __future__ import annotations

import ctypes
import os

PROBE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflce_probe.so")
EXPORTED = ("flce_probe_mfma_stream", "flce_probe_mfma_flops")
_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_PATH):
            raise RuntimeError(f"{PROBE_PATH} is not built: run "
                               "`python -m linear_cross_entropy_02_amd.build`")
        lib = ctypes.CDLL(PROBE_PATH)
        lib.flce_probe_mfma_stream.restype = ctypes.c_int32
        lib.flce_probe_mfma_stream.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p] * 2
        lib.flce_probe_mfma_flops.restype = ctypes.c_double
        lib.flce_probe_mfma_flops.argtypes = [ctypes.c_int32] * 3
        _lib = lib
    return _lib


def mfma_flops(shape: int, blocks: int, iters: int) -> float:
    return load().flce_probe_mfma_flops(shape, blocks, iters)


def mfma_stream(shape: int, blocks: int, iters: int, random_operands: bool, sink, stream=None):
    """Enqueue one probe launch; `sink` is a float32 CUDA tensor of at least
    blocks*256 elements (the per-thread accumulator sums land there)."""
    import torch
    if sink.dtype != torch.float32 or not sink.is_cuda or sink.numel() < blocks * 256:
        raise ValueError("sink must be a float32 device tensor of blocks*256 elements")
    s = stream if stream is not None else torch.cuda.current_stream()
    rc = load().flce_probe_mfma_stream(shape, blocks, iters, int(bool(random_operands)),
                                       ctypes.c_void_p(sink.data_ptr()),
                                       ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"flce_probe_mfma_stream failed ({rc})")
