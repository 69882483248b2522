"""Float64 CPU oracle for the fused linear cross-entropy head.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only tests, the smoke check and the benchmark's CPU
baseline leg do.  It shares no code with the HIP library.

What it computes, written out plainly from the pages (sources cited per
function by page title and section):

  z_tv   = sum_h X_th W_vh                       (logits = X @ W^T)
  m_t    = max_v z_tv
  lse_t  = m_t + ln sum_v exp(z_tv - m_t)        (stable logsumexp, two passes)
  valid_t = [y_t != ignore_index]
  l_t    = valid_t (lse_t - z_{t, y_t})          (NLL of log-softmax)
  loss   = sum_t l_t / n_valid   (mean)  or  sum_t l_t  (sum)
  s      = 1 / n_valid           (mean)  or  1          (sum)
  dZ_tv  = s valid_t (exp(z_tv - lse_t) - [v = y_t])
  dX     = dZ W,    dW = dZ^T X
  argmax_t = smallest v with z_tv = m_t

Readings where the pages are silent:
  * mean with n_valid = 0 returns loss 0 and zero gradients (the literal
    masked mean would be 0/0);
  * lse and argmax are reported for every row, ignored or not (they depend
    only on X and W);
  * a target outside [0, V) that is not ignore_index is an error here.

All arithmetic is float64 on the exact input values (bf16 or fp32 inputs are
upcast without rounding).  The token loop processes `chunk` rows at a time so
that no T x V float64 array is ever held; the chunking does not change the
mathematics (each row's softmax is independent, dW is a plain sum over rows).
"""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np

__all__ = ["flce_reference", "flce_bruteforce", "flce_rows", "flce_dw_rows", "validity",
           "count_valid", "scale_factor", "distill_reference", "distill_bruteforce"]


def validity(y: np.ndarray, ignore_index: int) -> np.ndarray:
    """valid_t = [y_t != ignore_index].

    Alisa's book of LLMs, Mathy things > Information theory > implementing the
    loss: tokens equal to the padding index are masked out of the loss.
    """
    return np.asarray(y) != ignore_index


def count_valid(y: np.ndarray, ignore_index: int) -> int:
    """n_valid = mask.sum() (same section: the masked mean divides by it)."""
    return int(validity(y, ignore_index).sum())


def scale_factor(n_valid: int, reduction: str) -> float:
    """Seed of the backward pass for the chosen reduction.

    Alisa's book of LLMs, Backpropagation: backward is seeded with 1 and, for
    a mean over per-token losses, linearity gives each token a factor
    1/n.  Reading: n_valid = 0 under mean gives 0 (no NaN).
    """
    if reduction == "sum":
        return 1.0
    if reduction != "mean":
        raise ValueError(reduction)
    return 0.0 if n_valid == 0 else 1.0 / n_valid


def _check_targets(y: np.ndarray, V: int, ignore_index: int) -> None:
    valid = validity(y, ignore_index)
    bad = valid & ((y < 0) | (y >= V))
    if bad.any():
        raise ValueError(f"{int(bad.sum())} target(s) outside [0, {V})")


def flce_reference(X: np.ndarray, W: np.ndarray, y: np.ndarray,
                   ignore_index: int = -100, reduction: str = "mean",
                   chunk: int = 1024, want_grads: bool = True) -> Dict[str, np.ndarray]:
    """Loss, per-token lse, argmax/top-2 gap, dX and dW in float64.

    Steps, in the pages' order:
      1. logits z = X W^T -- Alisa's book of LLMs, Neural net basics >
         Multi-layer perceptrons (PyTorch stores W as (out, in) and the
         forward multiplies by its transpose); efficient-llm-anatomy,
         Selected insights > Fused cross-entropy computes backward during
         forward (the three matmuls per token chunk).
      2. stable logsumexp, max first and then the shifted sum --
         Alisa's book of LLMs, Numerical stability and other tricks.
      3. NLL of log-softmax = z - lse, masked mean --
         Alisa's book of LLMs, Mathy things > Information theory.
      4. dZ = softmax - onehot(target), scaled and masked --
         Alisa's book of LLMs, gradient of softmax + CE loss; Backpropagation
         (mean seeds each token with 1/n).
      5. dX = dZ W (per-token activation grad) and dW = dZ^T X (parameter
         grad, summed over the batch) -- Alisa's book of LLMs, Neural net
         basics (batch rule for gradients: shared weights contract over the
         batch) and the efficient-llm-anatomy insight above.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    y = np.asarray(y, dtype=np.int64)
    T, H = X.shape
    V, H2 = W.shape
    if H2 != H or y.shape != (T,):
        raise ValueError("shape mismatch")
    _check_targets(y, V, ignore_index)
    valid = validity(y, ignore_index)
    n_valid = int(valid.sum())
    s = scale_factor(n_valid, reduction)

    lse = np.empty(T, dtype=np.float64)
    zmax = np.empty(T, dtype=np.float64)
    gap = np.full(T, np.inf, dtype=np.float64)
    amax = np.empty(T, dtype=np.int64)
    ztgt = np.zeros(T, dtype=np.float64)
    nll = np.zeros(T, dtype=np.float64)
    dX = np.zeros((T, H), dtype=np.float64) if want_grads else None
    dW = np.zeros((V, H), dtype=np.float64) if want_grads else None

    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        Xc = X[t0:t1]
        yc = y[t0:t1]
        vc = valid[t0:t1]
        Z = Xc @ W.T                                   # step 1
        m = Z.max(axis=1)                              # step 2, pass 1
        E = np.exp(Z - m[:, None])                     # step 2, pass 2
        l = m + np.log(E.sum(axis=1))
        lse[t0:t1] = l
        zmax[t0:t1] = m
        amax[t0:t1] = Z.argmax(axis=1)                 # first index of the max
        if V >= 2:
            top2 = np.partition(Z, V - 2, axis=1)[:, V - 2]
            gap[t0:t1] = m - top2
        rows = np.arange(t1 - t0)
        yv = np.where(vc, yc, 0)
        zt = np.where(vc, Z[rows, yv], 0.0)
        ztgt[t0:t1] = zt
        nll[t0:t1] = np.where(vc, l - zt, 0.0)         # step 3
        if want_grads:
            P = np.exp(Z - l[:, None])                 # step 4: softmax
            P[rows[vc], yc[vc]] -= 1.0                 #          - onehot
            dZ = P * (s * vc.astype(np.float64))[:, None]
            dX[t0:t1] = dZ @ W                         # step 5
            dW += dZ.T @ Xc
    total = float(nll.sum())
    loss = total * s if reduction == "mean" else total
    out = dict(loss=loss, lse=lse, zmax=zmax, argmax=amax, gap=gap,
               ztarget=ztgt, nll=nll, n_valid=n_valid, scale=s)
    if want_grads:
        out.update(dX=dX, dW=dW)
    return out


def flce_rows(X: np.ndarray, W: np.ndarray, y: np.ndarray, rows: Iterable[int],
              n_valid: int, ignore_index: int = -100, reduction: str = "mean",
              want_dx: bool = True, block: int = 8192) -> Dict[str, np.ndarray]:
    """Per-token outputs for a sample of rows.

    Same definitions as flce_reference, restricted to the listed rows; the
    global n_valid (a count over all targets, see count_valid) is passed in so
    that the mean's scale matches the full problem.  W is upcast to float64
    one block of vocabulary rows at a time, so full-size problems (W of
    several GB) are checked row-exactly without the complete oracle.
    """
    rows = np.array(list(rows), dtype=np.int64)
    V, H = W.shape
    s = scale_factor(n_valid, reduction)
    Xs = np.asarray(X[rows], dtype=np.float64)
    ys = np.asarray(y, dtype=np.int64)[rows]
    valid = validity(ys, ignore_index)
    if np.any(valid & ((ys < 0) | (ys >= V))):
        raise ValueError("target out of range")
    Z = np.empty((len(rows), V), dtype=np.float64)           # logits of the sample
    for v0 in range(0, V, block):
        Z[:, v0:v0 + block] = Xs @ np.asarray(W[v0:v0 + block], dtype=np.float64).T
    m = Z.max(axis=1)
    lse = m + np.log(np.exp(Z - m[:, None]).sum(axis=1))
    k = np.arange(len(rows))
    yv = np.where(valid, ys, 0)
    nll = np.where(valid, lse - Z[k, yv], 0.0)
    gap = (m - np.partition(Z, V - 2, axis=1)[:, V - 2]) if V >= 2 else np.full(len(rows), np.inf)
    res = dict(rows=rows, lse=lse, zmax=m, argmax=Z.argmax(axis=1), gap=gap, nll=nll,
               ztarget=np.where(valid, Z[k, yv], 0.0), scale=s, dX=None)
    if want_dx:
        P = np.exp(Z - lse[:, None])
        P[k[valid], ys[valid]] -= 1.0
        dZ = P * (s * valid.astype(np.float64))[:, None]
        dX = np.zeros((len(rows), H), dtype=np.float64)
        for v0 in range(0, V, block):
            dX += dZ[:, v0:v0 + block] @ np.asarray(W[v0:v0 + block], dtype=np.float64)
        res["dX"] = dX
    return res


def flce_dw_rows(X: np.ndarray, W: np.ndarray, y: np.ndarray, vrows: Iterable[int],
                 lse: np.ndarray, n_valid: int, ignore_index: int = -100,
                 reduction: str = "mean", block: int = 8192) -> np.ndarray:
    """Rows `vrows` of dW = dZ^T X, given every token's lse.

    Same definitions as flce_reference restricted to a sample of vocabulary
    rows: dZ_tv = s valid_t (exp(z_tv - lse_t) - [v = y_t]) for the listed v
    only (Alisa's book of LLMs, gradient of softmax + CE loss; Backpropagation
    for the mean's 1/n), and dW_v = sum_t dZ_tv X_t (Neural net basics, batch
    rule: the shared weight's gradient sums over the tokens).  `lse` is the
    oracle's own per-token lse over the whole vocabulary (flce_reference with
    want_grads=False), and n_valid the global count, so full-size problems
    are checked on their vocabulary rows without the T x V gradient.
    """
    vrows = np.array(list(vrows), dtype=np.int64)
    V, H = W.shape
    y = np.asarray(y, dtype=np.int64)
    lse = np.asarray(lse, dtype=np.float64)
    s = scale_factor(n_valid, reduction)
    valid = validity(y, ignore_index)
    if np.any(valid & ((y < 0) | (y >= V))):
        raise ValueError("target out of range")
    Wv = np.asarray(W[vrows], dtype=np.float64)                # [nv x H]
    out = np.zeros((len(vrows), H), dtype=np.float64)
    T = len(y)
    for t0 in range(0, T, block):
        t1 = min(T, t0 + block)
        Xb = np.asarray(X[t0:t1], dtype=np.float64)
        Z = Xb @ Wv.T                                          # z_tv, sampled v
        D = np.exp(Z - lse[t0:t1, None])
        D -= (y[t0:t1, None] == vrows[None, :])
        D *= (s * valid[t0:t1].astype(np.float64))[:, None]
        out += D.T @ Xb
    return out


def flce_bruteforce(X, W, y, ignore_index: int = -100, reduction: str = "mean") -> Dict[str, object]:
    """Pure-Python triple loops over the same definitions, for tiny inputs.

    No numpy arithmetic at all: every logit, exponential and product is a
    Python float operation, so a mistake in the vectorised oracle (a wrong
    axis, a broadcast, a transposed operand) cannot be shared by this one.
    """
    X = [[float(v) for v in row] for row in np.asarray(X)]
    W = [[float(v) for v in row] for row in np.asarray(W)]
    y = [int(v) for v in np.asarray(y)]
    T, V = len(X), len(W)
    H = len(X[0]) if T else len(W[0])
    valid = [yt != ignore_index for yt in y]
    n_valid = sum(valid)
    s = 1.0 if reduction == "sum" else (0.0 if n_valid == 0 else 1.0 / n_valid)
    dX = [[0.0] * H for _ in range(T)]
    dW = [[0.0] * H for _ in range(V)]
    lse, amax, total = [], [], 0.0
    for t in range(T):
        z = [sum(X[t][h] * W[v][h] for h in range(H)) for v in range(V)]
        m = max(z)
        l = m + math.log(sum(math.exp(zv - m) for zv in z))
        lse.append(l)
        amax.append(z.index(m))
        if not valid[t]:
            continue
        total += l - z[y[t]]
        for v in range(V):
            g = s * (math.exp(z[v] - l) - (1.0 if v == y[t] else 0.0))
            for h in range(H):
                dX[t][h] += g * W[v][h]
                dW[v][h] += g * X[t][h]
    loss = total * s if reduction == "mean" else total
    return dict(loss=loss, lse=lse, argmax=amax, dX=dX, dW=dW, n_valid=n_valid)


def loss_only(X, W, y, ignore_index: int = -100, reduction: str = "mean") -> float:
    """Scalar loss alone (used by finite-difference checks)."""
    return flce_reference(X, W, y, ignore_index, reduction, want_grads=False)["loss"]


# ---------------------------------------------------------------------------
# Soft-target (distillation) cross-entropy with a temperature.
#
#   z^S = X W^T (student),  z^T = X_T W_T^T (teacher, its own hidden size)
#   p_t = softmax(z^S_t / tau),  q_t = softmax(z^T_t / tau)
#   l_t = valid_t * H(q_t, p_t) = -valid_t sum_v q_tv ln p_tv
#   loss = s sum_t l_t,  dZ^S_tv = s valid_t (p_tv - q_tv) / tau
#   dX = dZ^S W,  dW = dZ^S^T X        (the teacher receives no gradient)
#
# Alisa's book of LLMs, Mathy things > Information theory: cross entropy of
# a target distribution against the model's is the KL divergence plus the
# target's own entropy, and for a one-hot target it is the NLL above;
# Neural net basics (softmax with temperature): logits are divided by the
# temperature before the softmax.  Readings: the targets array serves only
# as the mask (valid_t = [y_t != ignore_index]); no factor tau^2 is applied
# (a caller wanting the usual distillation scaling multiplies the loss and
# the gradients by tau^2); the gradient is the softmax + CE gradient of the
# same book (d/dz of -sum q ln softmax(z) = softmax(z) - q, since q sums to
# one) taken through the division by tau.
# ---------------------------------------------------------------------------
def distill_reference(X: np.ndarray, W: np.ndarray, X_teacher: np.ndarray,
                      W_teacher: np.ndarray, y: np.ndarray, ignore_index: int = -100,
                      temperature: float = 1.0, reduction: str = "mean",
                      chunk: int = 512, want_grads: bool = True) -> Dict[str, np.ndarray]:
    """Loss (and dX, dW of the student) of the soft-target CE above, float64."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    Xt = np.asarray(X_teacher, dtype=np.float64)
    Wt = np.asarray(W_teacher, dtype=np.float64)
    y = np.asarray(y)
    T, H = X.shape
    V = W.shape[0]
    if Xt.shape[0] != T or Wt.shape[0] != V or Xt.shape[1] != Wt.shape[1]:
        raise ValueError("teacher shapes")
    tau = float(temperature)
    if not tau > 0.0:
        raise ValueError("temperature must be positive")
    valid = validity(y, ignore_index)
    n_valid = int(valid.sum())
    s = scale_factor(n_valid, reduction)
    lse_s = np.zeros(T)
    lse_t = np.zeros(T)
    per_token = np.zeros(T)
    dX = np.zeros((T, H)) if want_grads else None
    dW = np.zeros((V, H)) if want_grads else None
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        a = (X[t0:t1] @ W.T) / tau                     # student logits / tau
        b = (Xt[t0:t1] @ Wt.T) / tau                   # teacher logits / tau
        ma = a.max(axis=1)
        la = ma + np.log(np.exp(a - ma[:, None]).sum(axis=1))
        mb = b.max(axis=1)
        lb = mb + np.log(np.exp(b - mb[:, None]).sum(axis=1))
        lse_s[t0:t1] = la
        lse_t[t0:t1] = lb
        logp = a - la[:, None]                         # log-softmax, student
        q = np.exp(b - lb[:, None])                    # softmax, teacher
        vc = valid[t0:t1]
        per_token[t0:t1] = np.where(vc, -(q * logp).sum(axis=1), 0.0)
        if want_grads:
            g = (np.exp(logp) - q) * (s * vc.astype(np.float64) / tau)[:, None]
            dX[t0:t1] = g @ W
            dW += g.T @ X[t0:t1]
    total = float(per_token.sum())
    loss = total * s if reduction == "mean" else total
    out = dict(loss=loss, per_token=per_token, lse_student=lse_s, lse_teacher=lse_t,
               n_valid=n_valid, scale=s)
    if want_grads:
        out.update(dX=dX, dW=dW)
    return out


def distill_bruteforce(X, W, X_teacher, W_teacher, y, ignore_index: int = -100,
                       temperature: float = 1.0, reduction: str = "mean") -> Dict[str, object]:
    """Pure-Python loops over the same definitions, for tiny inputs."""
    X = [[float(v) for v in row] for row in np.asarray(X)]
    W = [[float(v) for v in row] for row in np.asarray(W)]
    Xt = [[float(v) for v in row] for row in np.asarray(X_teacher)]
    Wt = [[float(v) for v in row] for row in np.asarray(W_teacher)]
    y = [int(v) for v in np.asarray(y)]
    T, V, H = len(X), len(W), len(X[0])
    Ht = len(Xt[0])
    tau = float(temperature)
    valid = [yt != ignore_index for yt in y]
    n_valid = sum(valid)
    s = 1.0 if reduction == "sum" else (0.0 if n_valid == 0 else 1.0 / n_valid)
    dX = [[0.0] * H for _ in range(T)]
    dW = [[0.0] * H for _ in range(V)]
    total = 0.0
    for t in range(T):
        if not valid[t]:
            continue
        a = [sum(X[t][h] * W[v][h] for h in range(H)) / tau for v in range(V)]
        b = [sum(Xt[t][h] * Wt[v][h] for h in range(Ht)) / tau for v in range(V)]
        za = sum(math.exp(x - max(a)) for x in a)
        zb = sum(math.exp(x - max(b)) for x in b)
        p = [math.exp(x - max(a)) / za for x in a]
        q = [math.exp(x - max(b)) / zb for x in b]
        total += -sum(q[v] * math.log(p[v]) for v in range(V))
        for v in range(V):
            g = s * (p[v] - q[v]) / tau
            for h in range(H):
                dX[t][h] += g * W[v][h]
                dW[v][h] += g * X[t][h]
    loss = total * s if reduction == "mean" else total
    return dict(loss=loss, dX=dX, dW=dW, n_valid=n_valid)
