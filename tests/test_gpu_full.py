"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.

For each large workload the float64 oracle's forward runs over every token
(blocks of tokens, progress printed), so the loss, every lse and every
argmax are compared with the oracle itself.  The gradients are compared on
samples the oracle computes one by one:
  * dX on sampled tokens (chunk boundaries, ignored tokens, random rows)
    against oracle.flce_rows;
  * dW on sampled vocabulary rows -- the most frequent targets, ids that are
    never a target, random ids, both vocabulary ends and, at 16384 x 4096 x
    128256, rows of the dW grid's last partial round (the tiles split three
    ways in K) -- against oracle.flce_dw_rows, given the oracle's own lse.
Both are checked per row as well as over the sample.  Properties that hold
at any size are checked on the whole tensors: ignored tokens have exactly
zero dX rows, n_valid is exact, the vocabulary sum of dW vanishes (every dZ
row sums to zero) and <dW, W> = <dX, X> (both equal sum_tv dZ_tv z_tv).
"""
import numpy as np
import pytest

import linear_cross_entropy_02_amd as flce
import workloads
from flce_check import LOSS_RTOL, LSE_ATOL, argmax_margin, check_argmax, check_grad, to_np
from oracle import count_valid, flce_dw_rows, flce_reference, flce_rows, scale_factor

pytestmark = pytest.mark.gpu

# each workload in the launch configuration the benchmark times
CHUNK = {n: workloads.launch_config(n) for n in (3, 4, 5)}


def log(msg):
    print(f"[gpu-full] {msg}", flush=True)


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


def sample_vocab_rows(V, y, ignore_index, seed, extra=()):
    """Frequent targets, never-targeted ids, random ids, both ends, extras."""
    rng = np.random.default_rng(seed)
    yv = y[(y != ignore_index) & (y >= 0)]
    counts = np.bincount(yv, minlength=V)
    frequent = np.argsort(-counts, kind="stable")[:8]
    never = np.nonzero(counts == 0)[0]
    rare = rng.choice(never, size=min(8, len(never)), replace=False) if len(never) else []
    vs = np.concatenate([frequent, rare, rng.choice(V, 16, replace=False), [0, V - 1],
                         np.asarray(list(extra), dtype=np.int64)])
    return np.unique(vs.astype(np.int64))


def run_full(cfg):
    import torch
    wl = workloads.WORKLOADS[cfg]
    log(f"generating workload {cfg}: {wl.name}")
    inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    chunk, g = CHUNK[cfg]
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=chunk, dw_chunks=g,
                                      weight_copy=workloads.weight_copy(cfg),
                                      dz_in_place=workloads.dz_in_place(cfg))
    log(f"workload {cfg} on GPU, chunk {op.chunk_tokens}, dw_chunks {op.dw_chunks}, "
        f"workspace {op.workspace_bytes / 2**20:.0f} MiB")
    out = op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction)
    torch.cuda.synchronize()
    # the workspace (with its logits-shaped buffers: the exponentials of the
    # G chunks of a dW group, or one chunk's and the group's dZ^T) stays
    # below a bf16 T x V buffer
    assert op.workspace_bytes < wl.T * wl.V * 2, (op.workspace_bytes, wl.T * wl.V * 2)
    res = {k: to_np(v) for k, v in out.items()}
    op.close()
    del X, W, y, out
    torch.cuda.empty_cache()
    log("GPU outputs copied to the host")
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
    return n_valid


def check_forward_against_oracle(wl, inp, res, block=4096):
    """The oracle's forward over every token, in blocks of tokens (each
    token's lse, argmax and NLL depend on that token alone); the loss is the
    oracle's NLL summed and scaled for the reduction."""
    T = wl.T
    W64 = np.asarray(inp.W, dtype=np.float64)
    lse = np.empty(T)
    zmax = np.empty(T)
    amax = np.empty(T, dtype=np.int64)
    nll = np.empty(T)
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        r = flce_reference(inp.X[t0:t1], W64, inp.y[t0:t1], wl.ignore_index, wl.reduction,
                           chunk=1024, want_grads=False)
        lse[t0:t1], zmax[t0:t1], amax[t0:t1], nll[t0:t1] = r["lse"], r["zmax"], r["argmax"], r["nll"]
        log(f"oracle forward: {t1} of {T} tokens")
    del W64
    n_valid = count_valid(inp.y, wl.ignore_index)
    loss = float(nll.sum()) * scale_factor(n_valid, wl.reduction)
    got = float(res["loss"])
    assert abs(got - loss) <= LOSS_RTOL * abs(loss), (got, loss)
    err = np.abs(res["lse"] - lse)
    assert err.max() <= LSE_ATOL, (int(err.argmax()), float(err.max()))
    delta = argmax_margin(inp.X, inp.W, np.arange(T))
    amb = check_argmax(res["argmax"], amax, zmax, inp.X, inp.W, np.arange(T), delta)
    log(f"loss {got:.6f} vs oracle {loss:.6f}; max lse error {err.max():.2e}; "
        f"argmax: {amb} rows inside the rounding margin")
    return lse, n_valid


def check_sampled_dx(wl, inp, res, n_valid, seed):
    rows = sample_rows(wl.T, CHUNK[wl_cfg(wl)][0], inp.y, wl.ignore_index, seed)
    log(f"oracle dX on {len(rows)} sampled rows")
    r = flce_rows(inp.X, inp.W, inp.y, rows, n_valid, wl.ignore_index, wl.reduction)
    assert np.abs(res["lse"][rows] - r["lse"]).max() <= LSE_ATOL
    e, er = check_grad("sampled dX", res["dX"][rows], r["dX"], wl.dtype)
    log(f"sampled dX: rel err {e:.2e}, worst row {er:.2e}")


def check_sampled_dw(wl, inp, res, lse, n_valid, seed, extra=()):
    vs = sample_vocab_rows(wl.V, inp.y, wl.ignore_index, seed, extra)
    log(f"oracle dW on {len(vs)} sampled vocabulary rows")
    want = flce_dw_rows(inp.X, inp.W, inp.y, vs, lse, n_valid, wl.ignore_index, wl.reduction)
    e, er = check_grad("sampled dW", res["dW"][vs], want, wl.dtype)
    log(f"sampled dW: rel err {e:.2e}, worst row {er:.2e}")


def wl_cfg(wl):
    return next(k for k, v in workloads.WORKLOADS.items() if v.name == wl.name)


def test_full_layer_model_shape():
    wl, inp, res = run_full(3)
    check_properties(wl, inp, res)
    lse, n_valid = check_forward_against_oracle(wl, inp, res, block=16384)
    check_sampled_dx(wl, inp, res, n_valid, seed=3)
    check_sampled_dw(wl, inp, res, lse, n_valid, seed=33)


def test_full_llama3_head():
    wl, inp, res = run_full(4)
    check_properties(wl, inp, res)
    lse, n_valid = check_forward_against_oracle(wl, inp, res)
    check_sampled_dx(wl, inp, res, n_valid, seed=4)
    # the dW grid (501 x 16 tiles) runs 31 full rounds of 256 tiles; its last
    # 80 tiles (vocabulary rows 126976 and up) are split three ways in K
    tail = np.random.default_rng(44).choice(np.arange(126976, wl.V), 8, replace=False)
    check_sampled_dw(wl, inp, res, lse, n_valid, seed=44, extra=tail)


def test_full_large_ragged_head():
    wl, inp, res = run_full(5)
    check_properties(wl, inp, res)
    lse, n_valid = check_forward_against_oracle(wl, inp, res)
    check_sampled_dx(wl, inp, res, n_valid, seed=5)
    # outlier rows of W (scaled x20) among the sampled dW rows
    outl = np.argsort(-np.abs(inp.W[:, :64]).max(axis=1))[:4]
    check_sampled_dw(wl, inp, res, lse, n_valid, seed=55, extra=outl)


def test_full_llama3_head_weight_as_stored_is_bitwise_equal():
    # dX reading W as stored adds the same products in the same order as
    # through the W^T copy, so at full size every output is the same bits
    import torch
    wl = workloads.WORKLOADS[4]
    log("generating workload 4 for the weight-copy comparison")
    inp = workloads.generate(wl, keep_f32=False)
    X, W, y = workloads.to_torch(inp, "cuda")
    chunk, g = CHUNK[4]
    outs = []
    for wcopy in (True, False):
        op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=chunk, dw_chunks=g,
                                          weight_copy=wcopy)
        log(f"workload 4, weight_copy {wcopy}, workspace {op.workspace_bytes / 2**20:.0f} MiB")
        outs.append(op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction))
        torch.cuda.synchronize()
        op.close()
    for k in ("loss", "dX", "dW", "lse", "argmax", "n_valid"):
        assert torch.equal(outs[0][k], outs[1][k]), k
