"""GPU parity of the forward-only entry point (flce_forward): per-token
log-probabilities of the targets, lse, argmax, n_valid and the reduced loss
against the float64 oracle, and agreement with flce_fwd_bwd's forward
outputs on the same inputs."""
import numpy as np
import pytest

import linear_cross_entropy_02_amd as flce
import workloads
from flce_check import LOSS_RTOL, LSE_ATOL, argmax_margin, check_argmax, to_np
from oracle import count_valid, flce_reference, flce_rows

pytestmark = pytest.mark.gpu

# per-token log-probs are z_target - lse: the same 1e-3 absolute bound as lse
LOGPROB_ATOL = 2 * LSE_ATOL


def check_forward(out, ref, inp, wl):
    loss = float(out["loss"].item())
    if ref["loss"] == 0.0:
        assert loss == 0.0
    else:
        assert abs(loss - ref["loss"]) <= LOSS_RTOL * abs(ref["loss"]), (loss, ref["loss"])
    assert int(out["n_valid"].item()) == ref["n_valid"]
    T = inp.X.shape[0]
    if not T:
        return
    ign = inp.y == wl.ignore_index
    lp = to_np(out["token_logprob"])
    assert np.all(lp[ign] == 0.0), "ignored tokens must have log-prob exactly 0"
    assert np.all(lp[~ign] <= 1e-6), "log-probabilities are not positive"
    # the oracle's per-token NLL is valid_t (lse_t - z_{t, y_t})
    assert np.abs(lp - (-ref["nll"])).max() <= LOGPROB_ATOL, np.abs(lp + ref["nll"]).max()
    lse = to_np(out["lse"])
    assert np.abs(lse - ref["lse"]).max() <= LSE_ATOL
    rows = np.arange(T)
    check_argmax(to_np(out["argmax"]), ref["argmax"], ref["zmax"], inp.X, inp.W, rows,
                 argmax_margin(inp.X, inp.W, rows))


CASES = [
    (workloads.WORKLOADS[1], 0),
    (workloads.WORKLOADS[1].with_shape(T=200, V=777, seed=51), 64),
    (workloads.WORKLOADS[2].with_shape(T=1000, H=96, V=1000, seed=52), 256),
    (workloads.WORKLOADS[4].with_shape(T=600, H=1024, V=20000, seed=53), 256),
    (workloads.WORKLOADS[5].with_shape(T=700, H=512, V=12345, seed=54), 256),
]


@pytest.mark.parametrize("wl,chunk", CASES, ids=[c[0].name for c in CASES])
def test_forward_vs_oracle(wl, chunk):
    import torch
    inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=chunk)
    print(f"[gpu-forward] {wl.name} T={wl.T} H={wl.H} V={wl.V} chunk={op.chunk_tokens}",
          flush=True)
    out = op.forward(X, W, y, wl.ignore_index, wl.reduction)
    torch.cuda.synchronize()
    ref = flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction, want_grads=False)
    check_forward(out, ref, inp, wl)
    op.close()


def test_forward_matches_fwd_bwd_bitwise():
    """Same logits GEMM and epilogue arithmetic: lse, argmax and loss of the
    forward-only call equal those of the fused forward+backward exactly."""
    import torch
    wl = workloads.WORKLOADS[4].with_shape(T=900, H=512, V=20000, seed=55)
    inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=256)
    full = op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction)
    fwd = op.forward(X, W, y, wl.ignore_index, wl.reduction)
    torch.cuda.synchronize()
    assert torch.equal(full["lse"], fwd["lse"])
    assert torch.equal(full["argmax"], fwd["argmax"])
    assert torch.equal(full["loss"], fwd["loss"])
    assert torch.equal(full["n_valid"], fwd["n_valid"])
    op.close()


def test_forward_empty_and_all_ignored():
    import torch
    wl = workloads.WORKLOADS[2].with_shape(T=300, H=128, V=1000, seed=56)
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, "bf16")
    inp = workloads.generate(wl)
    inp.y[:] = wl.ignore_index
    X, W, y = workloads.to_torch(inp, "cuda")
    out = op.forward(X, W, y, wl.ignore_index, "mean")
    torch.cuda.synchronize()
    assert float(out["loss"].item()) == 0.0 and int(out["n_valid"].item()) == 0
    assert torch.all(out["token_logprob"] == 0).item()
    # T = 0: only the scalars are written
    loss = torch.full((), 7.0, device="cuda")
    nv = torch.full((), 7, dtype=torch.int64, device="cuda")
    st = flce.flce_forward(op.handle, None, W, None, 0, -100, flce.FLCE_SUM, loss, None, None,
                           None, nv)
    assert st == flce.FLCE_OK
    torch.cuda.synchronize()
    assert float(loss.item()) == 0.0 and int(nv.item()) == 0
    op.close()


def test_forward_out_of_range_targets_and_arguments():
    import torch
    wl = workloads.WORKLOADS[2].with_shape(T=256, H=64, V=400, seed=57)
    inp = workloads.generate(wl)
    y_bad = inp.y.copy()
    y_bad[[3, 50]] = [wl.V, -5]
    X, W, y = workloads.to_torch(workloads.Inputs(wl, inp.X, inp.W, y_bad, inp.x_bits,
                                                  inp.w_bits), "cuda")
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, "bf16")
    out = op.forward(X, W, y, wl.ignore_index, wl.reduction)
    st, bad = flce.flce_query_error(op.handle)
    assert st == flce.FLCE_ERR_BAD_TARGET and bad == 2
    lp = to_np(out["token_logprob"])
    assert lp[3] == 0.0 and lp[50] == 0.0
    # argument errors return before any work
    h = op.handle
    assert flce.flce_forward(h, X, W, y, -1, -100, flce.FLCE_MEAN) == flce.FLCE_ERR_INVALID_ARGUMENT
    assert flce.flce_forward(h, X, W, y, wl.T, -100, 3) == flce.FLCE_ERR_INVALID_ARGUMENT
    assert flce.flce_forward(h, X, None, y, wl.T, -100, flce.FLCE_MEAN) == \
        flce.FLCE_ERR_INVALID_ARGUMENT
    assert flce.flce_forward(h, None, W, y, wl.T, -100, flce.FLCE_MEAN) == \
        flce.FLCE_ERR_INVALID_ARGUMENT
    op.close()


def test_forward_full_size_llama_head():
    """The Llama-3-8B head (T=16384, H=4096, V=128256) at full size in the
    benchmark's chunking: sampled rows
    against the oracle's per-row outputs, and the loss against the mean of
    the per-token log-probs."""
    import torch
    wl = workloads.WORKLOADS[4]
    print(f"[gpu-forward] full {wl.name}", flush=True)
    inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=4096)
    out = op.forward(X, W, y, wl.ignore_index, wl.reduction)
    torch.cuda.synchronize()
    lp = to_np(out["token_logprob"])
    ign = inp.y == wl.ignore_index
    assert np.all(lp[ign] == 0.0) and np.isfinite(lp).all()
    n_valid = count_valid(inp.y, wl.ignore_index)
    assert int(out["n_valid"].item()) == n_valid
    loss = float(out["loss"].item())
    assert abs(loss - (-lp.sum() / n_valid)) <= LOSS_RTOL * abs(loss)
    rng = np.random.default_rng(58)
    rows = np.unique(np.concatenate([rng.choice(wl.T, 40, replace=False),
                                     [0, 4095, 4096, wl.T - 1], np.nonzero(ign)[0][:4]]))
    ref = flce_rows(inp.X, inp.W, inp.y, rows, n_valid, wl.ignore_index, wl.reduction,
                    want_dx=False)
    assert np.abs(to_np(out["lse"])[rows] - ref["lse"]).max() <= LSE_ATOL
    assert np.abs(lp[rows] + ref["nll"]).max() <= LOGPROB_ATOL
    check_argmax(to_np(out["argmax"])[rows], ref["argmax"], ref["zmax"], inp.X, inp.W, rows,
                 argmax_margin(inp.X, inp.W, rows))
    op.close()


@pytest.mark.parametrize("wl,chunk", [CASES[3], CASES[4]], ids=["zipf-head", "outlier-head"])
def test_forward_on_a_handle_without_the_weight_copy(wl, chunk):
    # the forward-only call never runs the dX contraction, so a handle that
    # reads W as stored (no W^T copy in its workspace) gives the same bits
    import torch
    inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    a = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=chunk)
    b = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=chunk, weight_copy=False)
    assert b.workspace_bytes < a.workspace_bytes
    ra = a.forward(X, W, y, wl.ignore_index, wl.reduction)
    rb = b.forward(X, W, y, wl.ignore_index, wl.reduction)
    torch.cuda.synchronize()
    for k in ra:
        assert torch.equal(ra[k], rb[k]), k
    a.close()
    b.close()


def test_forward_only_handle():
    """A handle made for the forward-only calls (FLCE_FLAG_FORWARD_ONLY):
    the same bits as a full handle's forward, a workspace of the merge's
    partials alone, a whole batch in one chunk, a vocabulary shard's
    forward step, and the backward entry points refused with nothing
    enqueued."""
    import torch
    wl = workloads.WORKLOADS[4].with_shape(T=3000, H=512, V=30000, seed=56)
    inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    full = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=1024)
    fo = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=1024, forward_only=True)
    nt = -(-wl.V // 128)
    print(f"[gpu-forward] forward-only handle: workspace {fo.workspace_bytes} against "
          f"{full.workspace_bytes}", flush=True)
    assert fo.workspace_bytes <= 12 * nt * 1024 + (64 << 10)
    a = full.forward(X, W, y, wl.ignore_index, wl.reduction)
    b = fo.forward(X, W, y, wl.ignore_index, wl.reduction)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    # the whole batch in one chunk: per-token results do not depend on the
    # chunking; the loss sums the same terms in another order
    one = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=3072, forward_only=True)
    c = one.forward(X, W, y, wl.ignore_index, wl.reduction)
    torch.cuda.synchronize()
    for k in ("token_logprob", "lse", "argmax", "n_valid"):
        assert torch.equal(a[k], c[k]), k
    assert abs(float(a["loss"].item()) - float(c["loss"].item())) <= 1e-6 * abs(float(a["loss"].item()))
    ref = flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction, want_grads=False)
    check_forward(c, ref, inp, wl)
    # step 1 of a vocabulary shard runs on it too, and matches a full handle's
    v0, v1 = 7000, 19000
    sa = flce.FusedLinearCrossEntropy(wl.H, v1 - v0, wl.dtype, chunk_tokens=1024)
    sb = flce.FusedLinearCrossEntropy(wl.H, v1 - v0, wl.dtype, chunk_tokens=1024,
                                      forward_only=True)
    Ws = W[v0:v1].contiguous()
    ra = sa.shard_forward(X, Ws, y, v0, wl.V, wl.ignore_index)
    rb = sb.shard_forward(X, Ws, y, v0, wl.V, wl.ignore_index)
    torch.cuda.synchronize()
    for k in ra:
        assert torch.equal(ra[k], rb[k]), k
    # the fused call and a shard's backward are refused before any work
    out = full.alloc_outputs(wl.T, "cuda")
    for t in out.values():
        t.fill_(7)
    torch.cuda.synchronize()
    st = flce.flce_fwd_bwd(fo.handle, X, W, y, wl.T, wl.ignore_index, flce.FLCE_MEAN,
                           out["loss"], out["dX"], out["dW"], out["lse"], out["argmax"],
                           out["n_valid"])
    assert st == flce.FLCE_ERR_INVALID_ARGUMENT
    with pytest.raises(flce.FlceError):
        sb.shard_backward(X, Ws, y, a["lse"], v0, wl.V, wl.ignore_index)
    torch.cuda.synchronize()
    assert float(out["loss"].item()) == 7.0
    for op in (full, fo, one, sa, sb):
        op.close()
