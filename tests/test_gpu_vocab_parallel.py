"""GPU parity of the vocabulary-parallel building blocks.

W is split by rows into uneven shards on one device; each shard runs
flce_vocab_shard_forward, the host merges the per-shard (max, sum of exp,
argmax, target logit) the way the collectives of a column-parallel lm_head
would (max, rescaled sum, sum), each shard then runs
flce_vocab_shard_backward with the merged lse, and the summed dX partials and
concatenated dW shards are compared with the float64 oracle on the whole W.
"""
import numpy as np
import pytest

import linear_cross_entropy_02_amd as flce
import workloads
from flce_check import GRAD_RTOL, LOSS_RTOL, LSE_ATOL, argmax_margin, check_argmax, rel_frob, to_np
from oracle import count_valid, flce_reference, scale_factor

pytestmark = pytest.mark.gpu


def run_sharded(wl, cuts, chunk=256, weight_copy=True, dw_chunks=0, dz_in_place=False):
    import torch
    inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    bounds = [0] + list(cuts) + [wl.V]
    print(f"[gpu-vocab-parallel] {wl.name} T={wl.T} H={wl.H} V={wl.V} shards {bounds}", flush=True)
    shards = []
    for v0, v1 in zip(bounds[:-1], bounds[1:]):
        op = flce.FusedLinearCrossEntropy(wl.H, v1 - v0, wl.dtype, chunk_tokens=chunk,
                                          dw_chunks=dw_chunks, weight_copy=weight_copy,
                                          dz_in_place=dz_in_place)
        Ws = W[v0:v1].contiguous()
        part = op.shard_forward(X, Ws, y, v0, wl.V, wl.ignore_index)
        shards.append((op, v0, Ws, {k: to_np(v) for k, v in part.items()}))
    torch.cuda.synchronize()
    # the caller's collectives, in float64 on the host
    m = np.stack([p["m"] for _, _, _, p in shards])
    se = np.stack([p["sumexp"] for _, _, _, p in shards])
    M = m.max(axis=0)
    lse = M + np.log((se * np.exp(m - M)).sum(axis=0))
    zt = np.stack([p["ztarget"] for _, _, _, p in shards]).sum(axis=0)
    first = np.argmax(m == M, axis=0)     # lowest shard holding the max: lowest ids
    amax = np.stack([p["argmax"] for _, _, _, p in shards])[first, np.arange(wl.T)]
    valid = inp.y != wl.ignore_index
    n_valid = count_valid(inp.y, wl.ignore_index)
    s = scale_factor(n_valid, wl.reduction)
    loss = s * float(np.where(valid, lse - zt, 0.0).sum())
    lse_dev = torch.tensor(lse, dtype=torch.float32, device="cuda")
    dX = np.zeros((wl.T, wl.H))
    dW = np.zeros((wl.V, wl.H))
    for op, v0, Ws, _ in shards:
        dXp, dWs = op.shard_backward(X, Ws, y, lse_dev, v0, wl.V, wl.ignore_index, wl.reduction)
        torch.cuda.synchronize()
        dX += to_np(dXp)
        dW[v0:v0 + Ws.shape[0]] = to_np(dWs)
        op.close()
    return inp, dict(loss=loss, lse=lse, argmax=amax, dX=dX, dW=dW)


CASES = [
    # (workload, shard boundaries, dX through a W^T copy)
    (workloads.WORKLOADS[4].with_shape(T=600, H=512, V=20000, seed=61), (7000, 13001)),
    (workloads.WORKLOADS[5].with_shape(T=700, H=256, V=12345, seed=62), (6000,)),
    (workloads.WORKLOADS[2].with_shape(T=1000, H=96, V=1000, seed=63), (100, 300, 999)),
    (workloads.WORKLOADS[1].with_shape(T=200, V=777, seed=64), (300,)),
]
CASES = [c + (True, 0, False) for c in CASES] + [
    # shards whose dX reads W_shard as stored
    (workloads.WORKLOADS[4].with_shape(T=600, H=512, V=20000, seed=65), (7000, 13001), False, 0,
     False),
    # each shard's dW over groups of chunks (5 chunks: groups of 2, 2, 1), with
    # dZ formed in the contractions and written in place
    (workloads.WORKLOADS[4].with_shape(T=1100, H=256, V=9000, seed=66), (4000,), False, 2, False),
    (workloads.WORKLOADS[4].with_shape(T=1100, H=256, V=9000, seed=67), (4000,), True, 2, True),
]


@pytest.mark.parametrize("wl,cuts,wcopy,g,in_place", CASES,
                         ids=[f"{c[0].name}-{len(c[1]) + 1}shards" + ("" if c[2] else "-no-wcopy") +
                              (f"-G{c[3]}" if c[3] else "") + ("-in-place" if c[4] else "")
                              for c in CASES])
def test_vocab_parallel_vs_oracle(wl, cuts, wcopy, g, in_place):
    inp, got = run_sharded(wl, cuts, weight_copy=wcopy, dw_chunks=g, dz_in_place=in_place)
    ref = flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction)
    assert abs(got["loss"] - ref["loss"]) <= LOSS_RTOL * abs(ref["loss"])
    assert np.abs(got["lse"] - ref["lse"]).max() <= LSE_ATOL
    rows = np.arange(wl.T)
    check_argmax(got["argmax"], ref["argmax"], ref["zmax"], inp.X, inp.W, rows,
                 argmax_margin(inp.X, inp.W, rows))
    tol = GRAD_RTOL[wl.dtype]
    assert rel_frob(got["dX"], ref["dX"]) <= tol
    assert rel_frob(got["dW"], ref["dW"]) <= tol
    assert np.all(got["dX"][inp.y == wl.ignore_index] == 0.0)


def test_shard_arguments_rejected():
    import torch
    op = flce.FusedLinearCrossEntropy(64, 300, "bf16")
    W = torch.zeros(300, 64, dtype=torch.bfloat16, device="cuda")
    X = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(8, dtype=torch.int64, device="cuda")
    f = [torch.empty(8, device="cuda") for _ in range(3)]
    a = torch.empty(8, dtype=torch.int32, device="cuda")
    bad = flce.FLCE_ERR_INVALID_ARGUMENT
    h = op.handle
    # shard past the end, negative offset, vocabulary smaller than the shard
    assert flce.flce_vocab_shard_forward(h, X, W, y, 8, -100, 1, 300, f[0], f[1], a, f[2]) == bad
    assert flce.flce_vocab_shard_forward(h, X, W, y, 8, -100, -1, 600, f[0], f[1], a, f[2]) == bad
    assert flce.flce_vocab_shard_forward(h, X, W, y, 8, -100, 0, 299, f[0], f[1], a, f[2]) == bad
    assert flce.flce_vocab_shard_forward(h, X, W, y, 8, -100, 0, 300, None, f[1], a, f[2]) == bad
    dX = torch.empty(8, 64, dtype=torch.bfloat16, device="cuda")
    dW = torch.empty(300, 64, device="cuda")
    assert flce.flce_vocab_shard_backward(h, X, W, y, 8, -100, 0, 600, flce.FLCE_MEAN, None, dX,
                                          dW) == bad
    assert flce.flce_vocab_shard_backward(h, X, W, y, 8, -100, 400, 600, flce.FLCE_MEAN, f[0],
                                          dX, dW) == bad
    op.close()
