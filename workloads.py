"""Seeded synthetic inputs for the fused linear cross-entropy head.

This module only draws numbers: hidden states X (T x H), an lm_head weight
W (V x H, nn.Linear layout), int64 targets y and the ignore mask.  It holds
none of the loss arithmetic, so both the float64 oracle (tests) and the HIP
path consume exactly the same bits from here.

Recipe (all draws use numpy PCG64; seed = 1000 + workload number, split with
SeedSequence(seed).spawn(4) into streams for X, W, targets, ignore mask):

* values are drawn in float32; for bf16 workloads they are rounded to bf16
  with round-to-nearest-even (bit arithmetic below, identical to torch's
  float32 -> bfloat16 conversion);
* X ~ N(0, 1); W ~ N(0, w_std^2); optional outlier rows of W (a seeded
  subset) are multiplied by a factor before rounding;
* targets are uniform over [0, V) or a truncated Zipf law
  P(y = k) ~ (k + 1)^-s, k in [0, V), sampled by inverse CDF (rank = id);
* an exact number round(frac * T) of tokens is set to ignore_index, either
  at seeded scattered positions or as contiguous runs whose lengths are
  uniform in [32, 512] (last run truncated) at seeded non-overlapping places.

The five named workloads are the fused-CE head shapes: a tiny fp32 case,
the efficient-llm-anatomy layer shape (B=4, S=1024, H=512, V=16000), its
full-model shape (B=16, S=4096), a Llama-3-8B-shaped head (H=4096,
V=128256) and a large ragged head (H=8192, V=128256, outlier rows, 25 %
ignored in runs, sum reduction).  LAUNCH records the chunking each of them
is timed and parity-tested in (a launch setting, not an input).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

IGNORE_INDEX = -100


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    V: int
    dtype: str                 # "f32" or "bf16"
    x_std: float = 1.0
    w_std: float = 0.02
    targets: str = "uniform"   # "uniform" | "zipf"
    zipf_s: float = 1.1
    ignore_frac: float = 0.0
    ignore_mode: str = "scatter"   # "scatter" | "runs"
    outlier_frac: float = 0.0      # fraction of W rows scaled by outlier_scale
    outlier_scale: float = 20.0
    reduction: str = "mean"        # "mean" | "sum"
    ignore_index: int = IGNORE_INDEX
    seed: int = 1000

    def with_shape(self, T=None, H=None, V=None, seed=None, name=None):
        return dataclasses.replace(
            self, T=self.T if T is None else T, H=self.H if H is None else H,
            V=self.V if V is None else V, seed=self.seed if seed is None else seed,
            name=name or f"{self.name}-T{T or self.T}-H{H or self.H}-V{V or self.V}")


WORKLOADS = {
    1: Workload("tiny-fp32", 128, 64, 512, "f32", w_std=0.05, ignore_frac=0.10,
                seed=1001),
    2: Workload("layer-B4S1024-H512-V16000", 4096, 512, 16000, "bf16", w_std=0.02,
                ignore_frac=0.05, seed=1002),
    3: Workload("model-B16S4096-H512-V16000", 65536, 512, 16000, "bf16", w_std=0.02,
                ignore_frac=0.05, seed=1003),
    4: Workload("llama3-8b-head-T16384-H4096-V128256", 16384, 4096, 128256, "bf16",
                w_std=0.02, targets="zipf", ignore_frac=0.02, seed=1004),
    5: Workload("large-ragged-T8192-H8192-V128256", 8192, 8192, 128256, "bf16",
                w_std=0.01, targets="zipf", ignore_frac=0.25, ignore_mode="runs",
                outlier_frac=0.001, reduction="sum", seed=1005),
}

# Launch configuration per workload: (tokens per chunk C, chunks per dW GEMM G),
# the fastest measured whose workspace stays below a bf16 T x V buffer.  The
# two chunk-sized buffers (exponentials of one chunk, dZ^T of G chunks) take
# (1 + G) C V elements.  At H = 4096, C = 2048 with G = 4 makes each dW GEMM
# 8192 tokens deep, so the dW tiles are written twice per call instead of
# four times.  The large ragged head (T = H = 8192) cannot stay below T x V
# (W^T alone is H V = T V elements there); it takes the fastest setting.
LAUNCH = {1: (256, 1), 2: (2048, 1), 3: (32768, 1), 4: (2048, 4), 5: (2048, 2)}
# The other entry points at the Llama-3-8B head's shape, chosen the same
# way: the forward-only call runs on a forward-only handle (the merge's
# partials are all its workspace; 8192-token chunks measured faster than
# 4096 and 16384); a vocabulary shard's head is V / N wide; the soft-target
# head also holds the teacher's chunk of exponentials.
LAUNCH_MODES = {"forward": (8192, 1), "shard": (4096, 1), "distill": (2048, 4)}


# Workloads whose handle reads W as stored in the dX GEMM instead of a
# transposed copy made per call: the 8192 x 8192 x 128256 head, where that
# copy alone is as large as a bf16 T x V buffer; the 4096 x 512 x 16000
# layer, where dropping it leaves room for 2048-token chunks under that bound
# (0.37 ms per step, against 0.42 with the copy and 1024-token chunks); and
# the 16384 x 4096 x 128256 head, where it takes the workspace from 0.79 to
# 0.56 of a bf16 T x V buffer for 1-2 % of the step time.
NO_WEIGHT_COPY = {2, 4, 5}
# The other entry points at the Llama-3-8B head's shape read W as stored as
# well: the forward-only call never runs the dX contraction (the copy would
# sit unused), and a vocabulary shard's head and the soft-target head measured
# 0.2-0.4 % slower per step for a quarter to a half of a bf16 T x V buffer less
# workspace.
NO_WEIGHT_COPY_MODES = {"forward", "shard", "distill"}


def weight_copy(n: int, mode: str = "fwd_bwd") -> bool:
    if mode != "fwd_bwd":
        return mode not in NO_WEIGHT_COPY_MODES
    return n not in NO_WEIGHT_COPY


# Workloads whose handle writes dZ out for the dX contraction
# (FLCE_FLAG_DZ_IN_PLACE) instead of forming it there: the outlier-row head,
# whose rows' tiles mostly lie far below the outlier tiles' power-of-two
# reference, so forming dZ in place of the exponentials' rewrite measured
# faster (39.8 against 41.2 ms per step).
DZ_IN_PLACE = {5}


def dz_in_place(n: int, mode: str = "fwd_bwd") -> bool:
    return mode == "fwd_bwd" and n in DZ_IN_PLACE


def launch_config(n: int, mode: str = "fwd_bwd") -> tuple[int, int]:
    if mode != "fwd_bwd":
        return LAUNCH_MODES[mode]
    return LAUNCH.get(n, (4096, 1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even; NaN kept quiet."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_f32(rng: np.random.Generator, shape, std: float, block_rows: int = 4096) -> np.ndarray:
    """N(0, std^2) float32, drawn row-block by row-block (bounded temporaries)."""
    out = np.empty(shape, dtype=np.float32)
    rows = shape[0]
    for r0 in range(0, rows, block_rows):
        r1 = min(rows, r0 + block_rows)
        rng.standard_normal(size=(r1 - r0,) + tuple(shape[1:]), dtype=np.float32, out=out[r0:r1])
    if std != 1.0:
        out *= np.float32(std)
    return out


def zipf_targets(rng: np.random.Generator, n: int, V: int, s: float) -> np.ndarray:
    """Truncated Zipf over ids [0, V): P(k) ~ (k+1)^-s, by inverse CDF."""
    w = np.arange(1, V + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    u = rng.random(n) * cdf[-1]
    y = np.searchsorted(cdf, u, side="right")
    return np.minimum(y, V - 1).astype(np.int64)


def ignore_positions(rng: np.random.Generator, T: int, frac: float, mode: str) -> np.ndarray:
    """Boolean mask of ignored tokens with exactly round(frac*T) entries set."""
    n = int(round(frac * T))
    mask = np.zeros(T, dtype=bool)
    if n <= 0:
        return mask
    if mode == "scatter":
        mask[rng.choice(T, size=n, replace=False)] = True
        return mask
    if mode != "runs":
        raise ValueError(mode)
    lengths = []
    total = 0
    while total < n:
        L = int(rng.integers(32, 513))
        L = min(L, n - total)
        lengths.append(L)
        total += L
    r = len(lengths)
    free = T - n
    # stars and bars: r sorted gaps in [0, free], runs placed in order
    slots = np.sort(rng.choice(free + r, size=r, replace=False))
    gaps = slots - np.arange(r)
    start_base = 0
    for i, L in enumerate(lengths):
        s = int(gaps[i]) + start_base
        mask[s:s + L] = True
        start_base += L
    assert int(mask.sum()) == n
    return mask


@dataclasses.dataclass
class Inputs:
    """Host copies of one workload's inputs.

    X, W are float32 arrays holding exactly representable values of the
    workload dtype (bf16 values for bf16 workloads); x_bits / w_bits hold the
    bf16 bit patterns (uint16) when dtype == "bf16".
    """
    wl: Workload
    X: np.ndarray
    W: np.ndarray
    y: np.ndarray
    x_bits: Optional[np.ndarray] = None
    w_bits: Optional[np.ndarray] = None


def generate(wl: Workload, keep_f32: bool = True) -> Inputs:
    ss = np.random.SeedSequence(wl.seed).spawn(4)
    rx, rw, ry, rm = (np.random.Generator(np.random.PCG64(s)) for s in ss)
    X = _normal_f32(rx, (wl.T, wl.H), wl.x_std)
    W = _normal_f32(rw, (wl.V, wl.H), wl.w_std)
    if wl.outlier_frac > 0:
        n_out = int(round(wl.outlier_frac * wl.V))
        rows = rw.choice(wl.V, size=n_out, replace=False)
        W[rows] *= np.float32(wl.outlier_scale)
    if wl.targets == "uniform":
        y = ry.integers(0, wl.V, size=wl.T, dtype=np.int64)
    elif wl.targets == "zipf":
        y = zipf_targets(ry, wl.T, wl.V, wl.zipf_s)
    else:
        raise ValueError(wl.targets)
    mask = ignore_positions(rm, wl.T, wl.ignore_frac, wl.ignore_mode)
    y[mask] = wl.ignore_index
    if wl.dtype == "f32":
        return Inputs(wl, X, W, y)
    if wl.dtype != "bf16":
        raise ValueError(wl.dtype)
    xb = f32_to_bf16_bits(X)
    wb = f32_to_bf16_bits(W)
    if keep_f32:
        X = bf16_bits_to_f32(xb)
        W = bf16_bits_to_f32(wb)
        return Inputs(wl, X, W, y, xb, wb)
    return Inputs(wl, None, None, y, xb, wb)


def to_torch(inp: Inputs, device="cuda"):
    """(X, W, y) as torch tensors on `device` in the workload dtype."""
    import torch
    if inp.wl.dtype == "f32":
        X = torch.from_numpy(np.ascontiguousarray(inp.X)).to(device)
        W = torch.from_numpy(np.ascontiguousarray(inp.W)).to(device)
    else:
        X = torch.from_numpy(inp.x_bits.view(np.int16)).view(torch.bfloat16).to(device)
        W = torch.from_numpy(inp.w_bits.view(np.int16)).view(torch.bfloat16).to(device)
    y = torch.from_numpy(inp.y).to(device)
    return X, W, y
