"""Pins for the float64 oracle (CPU only).

The oracle is checked against things other than itself: a hand-worked
example, closed forms, invariants, finite differences, a pure-Python brute
force, PyTorch's own cross_entropy with autograd, and a statistical range.
Each pin is chosen so that a plausible slip (a dropped onehot term, a wrong
sign, a missing mask or scale, a transposed operand, an off-by-one target)
fails at least one of them; test_mutations plants such slips in the oracle
and checks that the pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest

import workloads
from oracle import flce_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_problem(T, H, V, seed, w_std=0.3, ignore_frac=0.25, ignore_index=-100):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, H))
    W = rng.standard_normal((V, H)) * w_std
    y = rng.integers(0, V, size=T)
    y[rng.random(T) < ignore_frac] = ignore_index
    return X, W, y


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    d = np.linalg.norm(a - b)
    n = np.linalg.norm(b)
    return d / n if n > 0 else d


# ---------------------------------------------------------------- golden ---
def test_golden_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_two_word_vocab.json")))
    X = np.array(g["X"])
    W = np.array([[0.0], [math.log(3.0)]])
    y = np.array(g["y"])
    e = g["expected"]
    for fn in (orc.flce_reference, orc.flce_bruteforce):
        r = fn(X, W, y, g["ignore_index"], g["reduction"])
        assert r["n_valid"] == e["n_valid"]
        assert abs(r["loss"] - e["loss"]) < 1e-14
        np.testing.assert_allclose(r["lse"], e["lse"], rtol=0, atol=1e-14)
        assert list(np.asarray(r["argmax"])) == e["argmax"]
        np.testing.assert_allclose(np.asarray(r["dX"]), e["dX"], rtol=0, atol=1e-15)
        np.testing.assert_allclose(np.asarray(r["dW"]), e["dW"], rtol=0, atol=1e-15)


# ---------------------------------------------------------- closed forms ---
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_p1_zero_weight_closed_form(reduction):
    T, H, V = 37, 5, 11
    X, _, y = rand_problem(T, H, V, 1)
    W = np.zeros((V, H))
    r = orc.flce_reference(X, W, y, -100, reduction, chunk=8)
    valid = y != -100
    n = int(valid.sum())
    assert np.all(r["lse"] == math.log(V))
    want = math.log(V) if reduction == "mean" else n * math.log(V)
    assert abs(r["loss"] - want) < 1e-12 * max(1, want)
    assert np.all(r["dX"] == 0.0)
    s = 1.0 / n if reduction == "mean" else 1.0
    dW = np.zeros((V, H))
    sum_valid = X[valid].sum(axis=0)
    for v in range(V):
        dW[v] = s * (sum_valid / V - X[valid & (y == v)].sum(axis=0))
    np.testing.assert_allclose(r["dW"], dW, rtol=0, atol=1e-13)
    assert np.all(r["argmax"] == 0)  # all ties: lowest index


def test_p5_two_word_vocab_is_logistic():
    """V = 2: NLL is softplus(-(z_y - z_other)), the logistic (BCE) loss."""
    T, H = 50, 7
    X, W, y = rand_problem(T, H, 2, 5, w_std=1.0, ignore_frac=0.0)
    r = orc.flce_reference(X, W, y, -100, "sum", chunk=16)
    Z = X @ W.T
    margin = Z[np.arange(T), y] - Z[np.arange(T), 1 - y]
    want = np.log1p(np.exp(-margin))
    np.testing.assert_allclose(r["nll"], want, rtol=1e-13, atol=1e-15)
    # gradient of softplus(-m): d/dz_y = -sigmoid(-m)
    sig = 1.0 / (1.0 + np.exp(margin))
    dz = np.zeros((T, 2))
    dz[np.arange(T), y] = -sig
    dz[np.arange(T), 1 - y] = sig
    np.testing.assert_allclose(r["dX"], dz @ W, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------ invariants ---
def test_p2_row_sum_invariant():
    X, W, y = rand_problem(64, 9, 23, 2)
    r = orc.flce_reference(X, W, y, chunk=10)
    # every dZ row sums to 0  =>  sum over vocab of dW is 0 for each h
    assert np.max(np.abs(r["dW"].sum(axis=0))) < 1e-14 * max(1.0, np.abs(r["dW"]).max()) * 23


def test_p3_ignored_tokens_contribute_nothing():
    X, W, y = rand_problem(40, 6, 13, 3, ignore_frac=0.3)
    ign = np.where(y == -100)[0]
    assert len(ign) > 0
    r = orc.flce_reference(X, W, y, chunk=7)
    assert np.all(r["dX"][ign] == 0.0)
    X2 = X.copy()
    X2[ign] += np.random.default_rng(9).standard_normal((len(ign), 6)) * 5
    r2 = orc.flce_reference(X2, W, y, chunk=7)
    assert r2["loss"] == pytest.approx(r["loss"], rel=1e-14, abs=1e-15)
    np.testing.assert_allclose(r2["dW"], r["dW"], rtol=1e-12, atol=1e-15)
    keep = np.setdiff1d(np.arange(40), ign)
    np.testing.assert_allclose(r2["dX"][keep], r["dX"][keep], rtol=1e-12, atol=1e-15)


def test_ignore_index_inside_vocab():
    """The padding index may be a real vocabulary id: equality decides."""
    X, W, y = rand_problem(30, 4, 9, 4, ignore_frac=0.0)
    y[::3] = 5
    r = orc.flce_reference(X, W, y, ignore_index=5)
    assert r["n_valid"] == int((y != 5).sum())
    assert np.all(r["dX"][y == 5] == 0.0)


def test_p8_mean_sum_relation():
    X, W, y = rand_problem(33, 5, 12, 6)
    rm = orc.flce_reference(X, W, y, -100, "mean")
    rs = orc.flce_reference(X, W, y, -100, "sum")
    n = rm["n_valid"]
    assert rs["loss"] == pytest.approx(n * rm["loss"], rel=1e-13)
    np.testing.assert_allclose(rs["dX"], n * rm["dX"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(rs["dW"], n * rm["dW"], rtol=1e-12, atol=1e-15)


def test_p9_permutations():
    X, W, y = rand_problem(24, 5, 10, 7)
    r = orc.flce_reference(X, W, y)
    rng = np.random.default_rng(1)
    pv = rng.permutation(10)          # new row i of W is old row pv[i]
    inv = np.argsort(pv)
    y2 = np.where(y == -100, -100, inv[np.where(y == -100, 0, y)])
    r2 = orc.flce_reference(X, W[pv], y2)
    assert r2["loss"] == pytest.approx(r["loss"], rel=1e-13)
    np.testing.assert_allclose(r2["lse"], r["lse"], rtol=1e-13)
    np.testing.assert_allclose(r2["dX"], r["dX"], rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(r2["dW"], r["dW"][pv], rtol=1e-11, atol=1e-15)
    pt = rng.permutation(24)
    r3 = orc.flce_reference(X[pt], W, y[pt])
    assert r3["loss"] == pytest.approx(r["loss"], rel=1e-13)
    np.testing.assert_allclose(r3["lse"], r["lse"][pt], rtol=1e-13)
    np.testing.assert_allclose(r3["dX"], r["dX"][pt], rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(r3["dW"], r["dW"], rtol=1e-11, atol=1e-15)


def test_p10_bounds():
    X, W, y = rand_problem(50, 8, 30, 8, w_std=2.0)
    r = orc.flce_reference(X, W, y)
    assert np.all(r["zmax"] <= r["lse"])
    assert np.all(r["lse"] <= r["zmax"] + math.log(30) + 1e-12)
    assert np.all(r["nll"] >= 0)


def test_stable_at_large_logits():
    """Shifting every logit of a row by a constant changes nothing (the
    stable-softmax argument); huge logits must not overflow."""
    T, H, V = 6, 3, 7
    X, W, y = rand_problem(T, H, V, 11, ignore_frac=0.0)
    r = orc.flce_reference(X, W, y)
    # append a hidden unit that adds 1000 to every logit of every row
    X2 = np.concatenate([X, np.full((T, 1), 1000.0)], axis=1)
    W2 = np.concatenate([W, np.ones((V, 1))], axis=1)
    r2 = orc.flce_reference(X2, W2, y)
    assert np.isfinite(r2["loss"])
    assert r2["loss"] == pytest.approx(r["loss"], rel=1e-12)
    np.testing.assert_allclose(r2["lse"], r["lse"] + 1000.0, rtol=1e-15)
    np.testing.assert_allclose(r2["dX"][:, :H], r["dX"], rtol=1e-9, atol=1e-13)


def test_chunking_does_not_change_results():
    X, W, y = rand_problem(70, 6, 17, 12)
    a = orc.flce_reference(X, W, y, chunk=1)
    b = orc.flce_reference(X, W, y, chunk=1000)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-14)
    np.testing.assert_allclose(a["dW"], b["dW"], rtol=1e-12, atol=1e-16)
    np.testing.assert_array_equal(a["argmax"], b["argmax"])


# ------------------------------------------------------------ edge cases ---
def test_empty_and_all_ignored():
    X = np.zeros((0, 4))
    W = np.random.default_rng(0).standard_normal((6, 4))
    r = orc.flce_reference(X, W, np.zeros(0, dtype=np.int64))
    assert r["loss"] == 0.0 and r["n_valid"] == 0
    assert r["dX"].shape == (0, 4) and np.all(r["dW"] == 0)
    X, W, y = rand_problem(10, 4, 6, 13, ignore_frac=1.1)
    assert np.all(y == -100)
    r = orc.flce_reference(X, W, y)
    assert r["loss"] == 0.0 and r["n_valid"] == 0
    assert np.all(r["dX"] == 0) and np.all(r["dW"] == 0)
    assert np.all(np.isfinite(r["lse"]))


def test_out_of_range_target_raises():
    X, W, y = rand_problem(5, 3, 4, 14, ignore_frac=0.0)
    y[2] = 4
    with pytest.raises(ValueError):
        orc.flce_reference(X, W, y)


def test_targets_at_vocab_ends():
    X, W, y = rand_problem(20, 4, 9, 15, ignore_frac=0.0)
    y[:10] = 0
    y[10:] = 8
    r = orc.flce_reference(X, W, y)
    b = orc.flce_bruteforce(X, W, y)
    assert r["loss"] == pytest.approx(b["loss"], rel=1e-13)
    np.testing.assert_allclose(r["dW"], np.array(b["dW"]), rtol=1e-11, atol=1e-15)


# ----------------------------------------------------- finite differences ---
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_p4_finite_differences(reduction):
    T, H, V = 7, 5, 11
    X, W, y = rand_problem(T, H, V, 16, w_std=0.7, ignore_frac=0.3)
    y[0] = 3  # at least one valid token
    r = orc.flce_reference(X, W, y, -100, reduction, chunk=3)
    h = 1e-6
    num_dX = np.zeros_like(X)
    for t in range(T):
        for k in range(H):
            Xp = X.copy(); Xp[t, k] += h
            Xm = X.copy(); Xm[t, k] -= h
            num_dX[t, k] = (orc.loss_only(Xp, W, y, -100, reduction) -
                            orc.loss_only(Xm, W, y, -100, reduction)) / (2 * h)
    num_dW = np.zeros_like(W)
    for v in range(V):
        for k in range(H):
            Wp = W.copy(); Wp[v, k] += h
            Wm = W.copy(); Wm[v, k] -= h
            num_dW[v, k] = (orc.loss_only(X, Wp, y, -100, reduction) -
                            orc.loss_only(X, Wm, y, -100, reduction)) / (2 * h)
    scale_x = np.abs(num_dX).max()
    scale_w = np.abs(num_dW).max()
    assert np.abs(r["dX"] - num_dX).max() < 1e-7 * scale_x
    assert np.abs(r["dW"] - num_dW).max() < 1e-7 * scale_w


# ------------------------------------------------------------ brute force ---
@pytest.mark.parametrize("seed,reduction", [(20, "mean"), (21, "sum"), (22, "mean")])
def test_p7_bruteforce(seed, reduction):
    X, W, y = rand_problem(9, 6, 13, seed)
    r = orc.flce_reference(X, W, y, -100, reduction, chunk=4)
    b = orc.flce_bruteforce(X, W, y, -100, reduction)
    assert r["n_valid"] == b["n_valid"]
    assert r["loss"] == pytest.approx(b["loss"], rel=1e-13, abs=1e-15)
    np.testing.assert_allclose(r["lse"], b["lse"], rtol=1e-14)
    np.testing.assert_array_equal(r["argmax"], b["argmax"])
    np.testing.assert_allclose(r["dX"], np.array(b["dX"]), rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(r["dW"], np.array(b["dW"]), rtol=1e-11, atol=1e-15)


# --------------------------------------------------------- library (torch) ---
@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_p6_torch_cross_entropy(reduction):
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    X, W, y = rand_problem(48, 16, 40, 23)
    r = orc.flce_reference(X, W, y, -100, reduction, chunk=13)
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(W, dtype=torch.float64, requires_grad=True)
    loss = F.cross_entropy(Xt @ Wt.T, torch.tensor(y), ignore_index=-100, reduction=reduction)
    loss.backward()
    lse = torch.logsumexp(Xt.detach() @ Wt.detach().T, dim=1).numpy()
    assert r["loss"] == pytest.approx(loss.item(), rel=1e-13)
    np.testing.assert_allclose(r["lse"], lse, rtol=1e-14)
    np.testing.assert_allclose(r["dX"], Xt.grad.numpy(), rtol=1e-11, atol=1e-16)
    np.testing.assert_allclose(r["dW"], Wt.grad.numpy(), rtol=1e-11, atol=1e-16)


@pytest.mark.parametrize("cfg", [1, 2])
def test_p6_torch_on_workloads(cfg):
    """The tiny fp32 head in full and a token slice of the 4096 x 512 x 16000
    layer shape, vs torch float64."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    wl = workloads.WORKLOADS[cfg]
    if cfg == 2:
        wl = wl.with_shape(T=512)
    inp = workloads.generate(wl)
    r = orc.flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction, chunk=256)
    Xt = torch.tensor(inp.X, dtype=torch.float64, requires_grad=True)
    Wt = torch.tensor(inp.W, dtype=torch.float64, requires_grad=True)
    loss = F.cross_entropy(Xt @ Wt.T, torch.tensor(inp.y), ignore_index=wl.ignore_index,
                           reduction=wl.reduction)
    loss.backward()
    assert r["loss"] == pytest.approx(loss.item(), rel=1e-12)
    assert rel_err(r["dX"], Xt.grad.numpy()) < 1e-12
    assert rel_err(r["dW"], Wt.grad.numpy()) < 1e-12


# ------------------------------------------------------------ row sampler ---
def test_rows_sampler_matches_full_oracle():
    wl = workloads.WORKLOADS[4].with_shape(T=96, H=64, V=3000, seed=77)
    inp = workloads.generate(wl)
    full = orc.flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction)
    rows = [0, 5, 17, 95]
    rr = orc.flce_rows(inp.X, inp.W, inp.y, rows, full["n_valid"], wl.ignore_index, wl.reduction)
    np.testing.assert_allclose(rr["lse"], full["lse"][rows], rtol=1e-13)
    np.testing.assert_allclose(rr["nll"], full["nll"][rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(rr["argmax"], full["argmax"][rows])
    np.testing.assert_allclose(rr["dX"], full["dX"][rows], rtol=1e-11, atol=1e-16)


def test_dw_row_sampler_matches_full_oracle():
    wl = workloads.WORKLOADS[4].with_shape(T=150, H=48, V=2500, seed=78)
    inp = workloads.generate(wl)
    full = orc.flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction)
    fwd = orc.flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction,
                             want_grads=False)
    vs = [0, 1, 7, int(inp.y[3]), 1999, 2499]
    got = orc.flce_dw_rows(inp.X, inp.W, inp.y, vs, fwd["lse"], full["n_valid"],
                           wl.ignore_index, wl.reduction, block=64)
    np.testing.assert_allclose(got, full["dW"][vs], rtol=1e-11, atol=1e-16)


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_dw_row_sampler_zero_weight_closed_form(reduction):
    # W = 0: every softmax is uniform and lse = ln V, so
    # dW_v = s (sum_{valid t} X_t / V - sum_{valid t, y_t = v} X_t)
    T, H, V = 41, 6, 13
    X, _, y = rand_problem(T, H, V, 3)
    W = np.zeros((V, H))
    valid = y != -100
    n = int(valid.sum())
    s = 1.0 / n if reduction == "mean" else 1.0
    vs = [0, 4, 12]
    got = orc.flce_dw_rows(X, W, y, vs, np.full(T, math.log(V)), n, -100, reduction, block=16)
    for k, v in enumerate(vs):
        want = s * (X[valid].sum(axis=0) / V - X[valid & (y == v)].sum(axis=0))
        np.testing.assert_allclose(got[k], want, rtol=0, atol=1e-13)


# ------------------------------------------------------- statistical range ---
@pytest.mark.parametrize("cfg,T,V", [(1, None, None), (2, None, None), (4, 64, 16384)])
def test_p11_expected_loss_range(cfg, T, V):
    """E[loss] ~ ln V + sigma_z^2 / 2 with sigma_z = sigma_W sqrt(H) for
    independent Gaussian X, W (a range check, not an exact pin)."""
    wl = workloads.WORKLOADS[cfg]
    if T is not None:
        wl = wl.with_shape(T=T, V=V)
    inp = workloads.generate(wl)
    r = orc.flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction,
                           chunk=1024, want_grads=False)
    expect = math.log(wl.V) + (wl.w_std ** 2) * wl.H / 2
    assert abs(r["loss"] - expect) / expect < 0.02


# -------------------------------------------------------------- mutations ---
def _mutated_reference(mutation):
    """A copy of the oracle's arithmetic with one planted slip."""
    def ref(X, W, y, ignore_index=-100, reduction="mean"):
        X = np.asarray(X, np.float64); W = np.asarray(W, np.float64)
        valid = y != ignore_index
        n = int(valid.sum())
        s = 1.0 if reduction == "sum" else 1.0 / n
        Z = X @ W.T
        m = Z.max(1)
        lse = m + np.log(np.exp(Z - m[:, None]).sum(1))
        rows = np.arange(len(y))
        yv = np.where(valid, y, 0)
        if mutation == "target_off_by_one":
            yv = np.minimum(yv + 1, W.shape[0] - 1)
        P = np.exp(Z - lse[:, None])
        if mutation != "drop_onehot":
            P[rows[valid], yv[valid]] -= 1.0
        mask = np.ones_like(valid) if mutation == "no_mask" else valid
        sc = 1.0 if mutation == "no_scale" else s
        sign = -1.0 if mutation == "sign" else 1.0
        dZ = sign * P * (sc * mask)[:, None]
        nll = np.where(valid, lse - Z[rows, yv], 0.0)
        loss = nll.sum() * (s if reduction == "mean" else 1.0)
        dX = dZ @ W
        dW = dZ.T @ X
        if mutation == "transpose":
            dW = (X.T @ dZ).T[::-1].copy()
        return dict(loss=loss, lse=lse, dX=dX, dW=dW, n_valid=n)
    return ref


@pytest.mark.parametrize("mutation", ["drop_onehot", "sign", "no_mask", "no_scale",
                                      "target_off_by_one", "transpose"])
def test_mutations_are_caught(mutation):
    """Each planted slip must fail at least one of the pins above."""
    bad = _mutated_reference(mutation)
    failures = 0
    # golden worked example
    g = json.load(open(os.path.join(GOLDEN, "worked_two_word_vocab.json")))
    W = np.array([[0.0], [math.log(3.0)]])
    r = bad(np.array(g["X"]), W, np.array(g["y"]))
    e = g["expected"]
    if (abs(r["loss"] - e["loss"]) > 1e-12 or
            np.abs(r["dX"] - np.array(e["dX"])).max() > 1e-12 or
            np.abs(r["dW"] - np.array(e["dW"])).max() > 1e-12):
        failures += 1
    # finite differences on dX
    X, Wm, y = rand_problem(5, 3, 6, 31, w_std=0.7, ignore_frac=0.3)
    y[0] = 2
    rb = bad(X, Wm, y)
    h = 1e-6
    num = np.zeros_like(X)
    for t in range(5):
        for k in range(3):
            Xp = X.copy(); Xp[t, k] += h
            Xm = X.copy(); Xm[t, k] -= h
            num[t, k] = (orc.loss_only(Xp, Wm, y) - orc.loss_only(Xm, Wm, y)) / (2 * h)
    if np.abs(rb["dX"] - num).max() > 1e-7 * np.abs(num).max():
        failures += 1
    # row-sum invariant and ignored-row pin
    if np.abs(rb["dW"].sum(0)).max() > 1e-12:
        failures += 1
    if np.any(rb["dX"][y == -100] != 0):
        failures += 1
    assert failures >= 1, f"mutation {mutation} slipped through every pin"
