"""GPU parity of the soft-target (distillation) path, flce_distill_fwd_bwd,
against the float64 distillation oracle."""
import numpy as np
import pytest

import linear_cross_entropy_02_amd as flce
import workloads
from flce_check import GRAD_RTOL, LOSS_RTOL, rel_frob, to_np
from oracle import distill_reference, flce_reference

pytestmark = pytest.mark.gpu


def run(wl, Ht, tau, chunk, teacher_seed, same_teacher=False, weight_copy=True, dw_chunks=0):
    import torch
    inp = workloads.generate(wl)
    if same_teacher:
        Xq_np, Wq_np = inp.X, inp.W
        X, W, y = workloads.to_torch(inp, "cuda")
        Xq, Wq = X, W
        Ht = wl.H
    else:
        tinp = workloads.generate(wl.with_shape(H=Ht, seed=teacher_seed))
        Xq_np, Wq_np = tinp.X, tinp.W
        X, W, y = workloads.to_torch(inp, "cuda")
        Xq, Wq, _ = workloads.to_torch(tinp, "cuda")
    op = flce.FusedDistillationCrossEntropy(wl.H, wl.V, Ht, wl.dtype, chunk_tokens=chunk,
                                            dw_chunks=dw_chunks, weight_copy=weight_copy)
    print(f"[gpu-distill] {wl.name} T={wl.T} H={wl.H} Ht={Ht} V={wl.V} tau={tau} "
          f"chunk={op.chunk_tokens} G={op.dw_chunks} wcopy={weight_copy}", flush=True)
    out = op.distill(X, W, Xq, Wq, y, tau, wl.ignore_index, wl.reduction)
    torch.cuda.synchronize()
    res = {k: to_np(v) for k, v in out.items()}
    op.close()
    ref = distill_reference(inp.X, inp.W, Xq_np, Wq_np, inp.y, wl.ignore_index, tau, wl.reduction)
    return inp, res, ref


CASES = [
    (workloads.WORKLOADS[2].with_shape(T=700, H=256, V=3000, seed=71), 128, 2.0, 256),
    (workloads.WORKLOADS[4].with_shape(T=600, H=512, V=20000, seed=72), 512, 1.0, 256),
    (workloads.WORKLOADS[5].with_shape(T=700, H=256, V=12345, seed=73), 384, 1.5, 256),
    (workloads.WORKLOADS[1], 32, 0.7, 0),
    (workloads.WORKLOADS[1].with_shape(T=200, V=777, seed=74), 48, 3.0, 64),
]
CASES = [c + (True, 0) for c in CASES] + [
    # the student's dX reading W as stored
    (workloads.WORKLOADS[4].with_shape(T=600, H=512, V=20000, seed=76), 512, 1.0, 256, False, 0),
    # dW over groups of chunks (5 chunks: groups of 2, 2 and 1), reading the
    # groups' dZ as stored (bf16) or through dZ^T (fp32)
    (workloads.WORKLOADS[4].with_shape(T=1100, H=512, V=20000, seed=77), 256, 1.2, 256, False, 2),
    (workloads.WORKLOADS[1].with_shape(T=300, V=777, seed=78), 48, 2.0, 64, True, 3),
]


@pytest.mark.parametrize("wl,Ht,tau,chunk,wcopy,g", CASES,
                         ids=[f"{c[0].name}-Ht{c[1]}-tau{c[2]}" + ("" if c[4] else "-no-wcopy") +
                              (f"-G{c[5]}" if c[5] else "") for c in CASES])
def test_distill_vs_oracle(wl, Ht, tau, chunk, wcopy, g):
    inp, res, ref = run(wl, Ht, tau, chunk, teacher_seed=wl.seed + 500, weight_copy=wcopy,
                        dw_chunks=g)
    assert abs(float(res["loss"]) - ref["loss"]) <= LOSS_RTOL * abs(ref["loss"]), \
        (float(res["loss"]), ref["loss"])
    assert int(res["n_valid"]) == ref["n_valid"]
    tol = GRAD_RTOL[wl.dtype]
    assert rel_frob(res["dX"], ref["dX"]) <= tol, rel_frob(res["dX"], ref["dX"])
    assert rel_frob(res["dW"], ref["dW"]) <= tol, rel_frob(res["dW"], ref["dW"])
    assert np.all(res["dX"][inp.y == wl.ignore_index] == 0.0)


def test_identical_teacher_gives_entropy_and_vanishing_gradient():
    wl = workloads.WORKLOADS[2].with_shape(T=500, H=256, V=3000, seed=75)
    inp, res, ref = run(wl, wl.H, 1.3, 256, teacher_seed=0, same_teacher=True)
    assert abs(float(res["loss"]) - ref["loss"]) <= LOSS_RTOL * abs(ref["loss"])
    hard = flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction)
    # p - q is bf16 rounding noise: tiny next to the one-hot gradient
    assert np.linalg.norm(res["dW"]) <= 1e-2 * np.linalg.norm(hard["dW"])
    assert np.linalg.norm(res["dX"]) <= 1e-2 * np.linalg.norm(hard["dX"])


def test_distill_arguments_rejected():
    import torch
    op = flce.FusedDistillationCrossEntropy(64, 300, 32, "bf16")
    plain = flce.FusedLinearCrossEntropy(64, 300, "bf16")
    X = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(300, 64, dtype=torch.bfloat16, device="cuda")
    Xq = torch.zeros(8, 32, dtype=torch.bfloat16, device="cuda")
    Wq = torch.zeros(300, 32, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(8, dtype=torch.int64, device="cuda")
    loss = torch.empty((), device="cuda")
    dX = torch.empty(8, 64, dtype=torch.bfloat16, device="cuda")
    dW = torch.empty(300, 64, device="cuda")
    bad = flce.FLCE_ERR_INVALID_ARGUMENT
    for tau in (0.0, -1.0, float("inf"), float("nan")):
        assert flce.flce_distill_fwd_bwd(op.handle, X, W, Xq, Wq, y, 8, -100, tau, flce.FLCE_MEAN,
                                         loss, dX, dW) == bad
    # a plain handle has no teacher buffers
    assert flce.flce_distill_fwd_bwd(plain.handle, X, W, Xq, Wq, y, 8, -100, 1.0, flce.FLCE_MEAN,
                                     loss, dX, dW) == bad
    assert flce.flce_distill_fwd_bwd(op.handle, X, W, None, Wq, y, 8, -100, 1.0, flce.FLCE_MEAN,
                                     loss, dX, dW) == bad
    op.close()
    plain.close()
