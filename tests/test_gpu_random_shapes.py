"""GPU parity on seeded random launch settings and shapes.

Each case draws T, H, V, the chunk size, the chunks per dW GEMM, the dtype,
the reduction, the share of ignored tokens, (bf16) whether dX reads a
transposed copy of W or W as stored, and whether dZ is written in place
(FLCE_FLAG_DZ_IN_PLACE), from its own seed, so the
combinations the hand-picked cases do not name (a batch shorter than one
chunk, a hidden size that is a multiple of 8 but not of 64, a vocabulary
below one tile, groups cut short by the batch) are compared with the
float64 oracle too.
"""
import dataclasses

import numpy as np
import pytest

import linear_cross_entropy_02_amd as flce
import workloads
from flce_check import check_full
from oracle import flce_reference

pytestmark = pytest.mark.gpu


def draw(seed):
    rng = np.random.default_rng(seed)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    vec = 4 if dtype == "f32" else 8
    T = int(rng.integers(1, 1500))
    H = int(vec * rng.integers(1, 520 // vec + 1))
    V = int(rng.integers(2, 5000))
    chunk = int(rng.choice([256, 512, 1024]))
    g = int(rng.integers(1, 4))
    base = workloads.WORKLOADS[1] if dtype == "f32" else workloads.WORKLOADS[2]
    wl = dataclasses.replace(
        base, name=f"random{seed}-{dtype}-T{T}-H{H}-V{V}-C{chunk}-G{g}", T=T, H=H, V=V,
        seed=5000 + seed, reduction=str(rng.choice(["mean", "sum"])),
        ignore_frac=float(rng.choice([0.0, 0.05, 0.3])))
    # from a stream of its own, so the draws above stay what they were
    wcopy = dtype == "f32" or bool(np.random.default_rng(seed + 7919).random() < 0.5)
    in_place = bool(np.random.default_rng(seed + 15485863).random() < 0.3)
    return wl, chunk, g, wcopy, in_place


@pytest.mark.parametrize("seed", list(range(96)))
def test_random_shape_vs_oracle(seed):
    import torch
    wl, chunk, g, wcopy, in_place = draw(seed)
    inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=chunk, dw_chunks=g,
                                      weight_copy=wcopy, dz_in_place=in_place)
    print(f"[gpu-random] {wl.name} {wl.reduction} ignore {wl.ignore_frac} weight_copy {wcopy} "
          f"dz_in_place {in_place}", flush=True)
    out = op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction)
    torch.cuda.synchronize()
    op.close()
    ref = flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction)
    check_full(out, ref, inp, wl)
