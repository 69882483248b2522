"""GPU parity at the full workload sizes.

The complete float64 oracle would take minutes here, so outputs are checked
(a) row-exactly on a seeded sample of tokens (chunk boundaries, ignored
tokens and random rows) against oracle.flce_rows, and (b) through properties
that hold at any size:
  * ignored tokens have exactly zero dX rows; n_valid is exact;
  * every dZ row sums to zero, so the vocabulary sum of dW vanishes;
  * <dW, W> = <dX, X> (both equal sum_tv dZ_tv z_tv);
  * loss = s sum_t valid_t (lse_t - z_{t, y_t}) with z_{t,y_t} = X_t . W_{y_t}.
The 65536 x 512 x 16000 model shape's forward (lse of every token) is
affordable on the host, so there the loss, every lse and a sample of dW
rows are compared exactly.
"""
import numpy as np
import pytest

import linear_cross_entropy_02_amd as flce
import workloads
from flce_check import LOSS_RTOL, LSE_ATOL, GRAD_RTOL, argmax_margin, check_argmax, rel_frob, to_np
from oracle import count_valid, flce_reference, flce_rows, scale_factor

pytestmark = pytest.mark.gpu

# each workload in the launch configuration the benchmark times
CHUNK = {n: workloads.launch_config(n) for n in (3, 4, 5)}


def sample_rows(T, C, y, ignore_index, seed, n=24):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    for c0 in range(0, T, C):
        rows.update({c0, min(T - 1, c0 + C - 1)})
    ign = np.nonzero(y == ignore_index)[0]
    if len(ign):
        rows.update(rng.choice(ign, size=min(4, len(ign)), replace=False).tolist())
    rows = sorted(rows)
    return np.array(rows[:64] if len(rows) > 64 else rows, dtype=np.int64)


def run_full(cfg):
    import torch
    wl = workloads.WORKLOADS[cfg]
    print(f"[gpu-full] generating workload {cfg}: {wl.name}", flush=True)
    inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    chunk, g = CHUNK[cfg]
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=chunk, dw_chunks=g,
                                      weight_copy=workloads.weight_copy(cfg))
    print(f"[gpu-full] workload {cfg} on GPU, chunk {op.chunk_tokens}, dw_chunks {op.dw_chunks}, "
          f"workspace {op.workspace_bytes / 2**20:.0f} MiB", flush=True)
    out = op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction)
    torch.cuda.synchronize()
    # the workspace holds logits-shaped chunk buffers of C x Vpad (exp / dZ)
    # and G C x Vpad (dZ^T of a dW group): together below T x V
    assert (1 + op.dw_chunks) * op.chunk_tokens < wl.T, "chunk buffers must stay below T x V"
    # and the whole workspace below a bf16 T x V buffer
    assert op.workspace_bytes < wl.T * wl.V * 2, (op.workspace_bytes, wl.T * wl.V * 2)
    res = {k: to_np(v) for k, v in out.items()}
    op.close()
    del X, W, y, out
    torch.cuda.empty_cache()
    return wl, inp, res


def check_properties(wl, inp, res):
    y = inp.y
    n_valid = count_valid(y, wl.ignore_index)
    assert int(res["n_valid"]) == n_valid
    s = scale_factor(n_valid, wl.reduction)
    valid = y != wl.ignore_index
    dX, dW = res["dX"], res["dW"]
    assert np.isfinite(dW).all() and np.isfinite(dX).all() and np.isfinite(res["lse"]).all()
    assert np.all(dX[~valid] == 0.0)
    # vocabulary sum of dW vanishes (relative to the size of either dZ term)
    colsum = dW.sum(axis=0, dtype=np.float64)
    ref_scale = s * np.linalg.norm(inp.X[valid].sum(axis=0, dtype=np.float64))
    assert np.linalg.norm(colsum) <= 2e-2 * ref_scale, (np.linalg.norm(colsum), ref_scale)
    # <dW, W> == <dX, X>
    a = b = 0.0
    for v0 in range(0, wl.V, 16384):
        a += float(np.sum(dW[v0:v0 + 16384] * inp.W[v0:v0 + 16384].astype(np.float64)))
    for t0 in range(0, wl.T, 8192):
        b += float(np.sum(dX[t0:t0 + 8192] * inp.X[t0:t0 + 8192].astype(np.float64)))
    assert abs(a - b) <= 1e-2 * max(abs(a), abs(b)), (a, b)
    # loss consistent with lse and the target logits
    yv = np.where(valid, y, 0)
    zt = np.einsum("th,th->t", inp.X.astype(np.float64), inp.W[yv].astype(np.float64))
    total = float(np.sum(np.where(valid, res["lse"].astype(np.float64) - zt, 0.0)))
    want = total * s if wl.reduction == "mean" else total
    assert abs(float(res["loss"]) - want) <= LOSS_RTOL * abs(want), (float(res["loss"]), want)
    return n_valid


def check_sampled_rows(wl, inp, res, n_valid, seed):
    rows = sample_rows(wl.T, CHUNK[wl_cfg(wl)][0], inp.y, wl.ignore_index, seed)
    print(f"[gpu-full] oracle on {len(rows)} sampled rows", flush=True)
    r = flce_rows(inp.X, inp.W, inp.y, rows, n_valid, wl.ignore_index, wl.reduction)
    assert np.abs(res["lse"][rows] - r["lse"]).max() <= LSE_ATOL
    e = rel_frob(res["dX"][rows], r["dX"])
    assert e <= GRAD_RTOL[wl.dtype], f"sampled dX rel err {e}"
    delta = argmax_margin(inp.X, inp.W, rows)
    check_argmax(res["argmax"][rows], r["argmax"], r["zmax"], inp.X, inp.W, rows, delta)


def wl_cfg(wl):
    return next(k for k, v in workloads.WORKLOADS.items() if v.name == wl.name)


def test_full_layer_model_shape():
    wl, inp, res = run_full(3)
    n_valid = check_properties(wl, inp, res)
    check_sampled_rows(wl, inp, res, n_valid, seed=3)
    # the whole forward is affordable on the host here
    print("[gpu-full] oracle forward over all tokens", flush=True)
    ref = flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction, chunk=2048,
                         want_grads=False)
    assert abs(float(res["loss"]) - ref["loss"]) <= LOSS_RTOL * abs(ref["loss"])
    assert np.abs(res["lse"] - ref["lse"]).max() <= LSE_ATOL
    # sampled dW rows: dW[v] = sum_t s valid_t (exp(z_tv - lse_t) - [y_t = v]) X_t
    rng = np.random.default_rng(33)
    vs = np.unique(np.concatenate([rng.choice(wl.V, 24, replace=False),
                                   inp.y[inp.y >= 0][:8], [0, wl.V - 1]]))
    X64 = inp.X.astype(np.float64)
    Zv = X64 @ inp.W[vs].astype(np.float64).T
    valid = inp.y != wl.ignore_index
    s = ref["scale"]
    P = np.exp(Zv - ref["lse"][:, None])
    P -= (inp.y[:, None] == vs[None, :])
    P *= (s * valid)[:, None]
    dWv = P.T @ X64
    e = rel_frob(res["dW"][vs], dWv)
    assert e <= GRAD_RTOL[wl.dtype], f"sampled dW rel err {e}"


def test_full_llama3_head():
    wl, inp, res = run_full(4)
    n_valid = check_properties(wl, inp, res)
    check_sampled_rows(wl, inp, res, n_valid, seed=4)


def test_full_large_ragged_head():
    wl, inp, res = run_full(5)
    n_valid = check_properties(wl, inp, res)
    check_sampled_rows(wl, inp, res, n_valid, seed=5)


def test_full_llama3_head_weight_as_stored_is_bitwise_equal():
    # dX reading W as stored adds the same products in the same order as
    # through the W^T copy, so at full size every output is the same bits
    import torch
    wl = workloads.WORKLOADS[4]
    print("[gpu-full] generating workload 4 for the weight-copy comparison", flush=True)
    inp = workloads.generate(wl, keep_f32=False)
    X, W, y = workloads.to_torch(inp, "cuda")
    chunk, g = CHUNK[4]
    outs = []
    for wcopy in (True, False):
        op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=chunk, dw_chunks=g,
                                          weight_copy=wcopy)
        print(f"[gpu-full] workload 4, weight_copy {wcopy}, workspace "
              f"{op.workspace_bytes / 2**20:.0f} MiB", flush=True)
        outs.append(op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction))
        torch.cuda.synchronize()
        op.close()
    for k in ("loss", "dX", "dW", "lse", "argmax", "n_valid"):
        assert torch.equal(outs[0][k], outs[1][k]), k
