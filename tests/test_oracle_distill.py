"""Pins of the soft-target (distillation) oracle against facts that do not
come from retyping its formula: the cross-entropy / KL / entropy identity
checked with scipy's entropy routines, the reduction to the hard-label CE
when the teacher is one-hot, the vanishing gradient when teacher and student
agree, finite differences and a pure-Python brute force."""
import numpy as np
import pytest
from scipy.special import rel_entr, softmax
from scipy.stats import entropy

from oracle import distill_bruteforce, distill_reference, flce_reference


def tiny(seed, T=6, H=4, Ht=3, V=7, ignore=(2,)):
    rng = np.random.default_rng(seed)
    X = rng.normal(size=(T, H))
    W = rng.normal(size=(V, H)) * 0.7
    Xt = rng.normal(size=(T, Ht))
    Wt = rng.normal(size=(V, Ht)) * 0.9
    y = rng.integers(0, V, size=T)
    y[list(ignore)] = -100
    return X, W, Xt, Wt, y


@pytest.mark.parametrize("tau", [1.0, 0.5, 2.5])
def test_identical_teacher_gives_entropy_and_zero_gradient(tau):
    X, W, _, _, y = tiny(1)
    ref = distill_reference(X, W, X, W, y, temperature=tau)
    valid = y != -100
    p = softmax((X @ W.T) / tau, axis=1)
    ent = np.array([entropy(p[t]) for t in range(len(y))])
    assert ref["loss"] == pytest.approx(ent[valid].mean(), rel=1e-12)
    assert np.abs(ref["dX"]).max() < 1e-14 and np.abs(ref["dW"]).max() < 1e-14


@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_one_hot_teacher_reduces_to_hard_label_ce(tau):
    """A teacher with a margin of 1000/tau at the label makes q one-hot, so
    the loss is the hard-label CE of softmax(z / tau): the pinned CE oracle
    on X / tau (its dX is with respect to X / tau, hence the 1 / tau)."""
    X, W, _, _, y = tiny(2, T=8, V=9, ignore=(0, 5))
    V = W.shape[0]
    yl = np.where(y == -100, 0, y)
    Xt = np.eye(V)[yl]
    Wt = 1000.0 * np.eye(V)
    d = distill_reference(X, W, Xt, Wt, y, temperature=tau)
    h = flce_reference(X / tau, W, y)
    assert d["loss"] == pytest.approx(h["loss"], rel=1e-12)
    np.testing.assert_allclose(d["dW"], h["dW"], rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(d["dX"], h["dX"] / tau, rtol=1e-10, atol=1e-14)


def test_cross_entropy_is_kl_plus_teacher_entropy():
    X, W, Xt, Wt, y = tiny(3, T=10, V=11)
    tau = 1.3
    d = distill_reference(X, W, Xt, Wt, y, temperature=tau, reduction="sum")
    p = softmax((X @ W.T) / tau, axis=1)
    q = softmax((Xt @ Wt.T) / tau, axis=1)
    valid = y != -100
    kl = rel_entr(q, p).sum(axis=1)
    hq = np.array([entropy(q[t]) for t in range(len(y))])
    assert d["loss"] == pytest.approx(float((kl + hq)[valid].sum()), rel=1e-12)
    assert np.all(d["per_token"][valid] >= hq[valid] - 1e-12)   # KL >= 0


def test_finite_differences():
    X, W, Xt, Wt, y = tiny(4, T=5, H=4, Ht=3, V=7, ignore=(1,))
    tau = 1.7
    ref = distill_reference(X, W, Xt, Wt, y, temperature=tau)
    eps = 1e-6

    def loss(Xa, Wa):
        return distill_reference(Xa, Wa, Xt, Wt, y, temperature=tau, want_grads=False)["loss"]

    for (arr, grad) in ((X, ref["dX"]), (W, ref["dW"])):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            a1 = arr.copy(); a1[idx] += eps
            a2 = arr.copy(); a2[idx] -= eps
            if arr is X:
                num[idx] = (loss(a1, W) - loss(a2, W)) / (2 * eps)
            else:
                num[idx] = (loss(X, a1) - loss(X, a2)) / (2 * eps)
        np.testing.assert_allclose(num, grad, rtol=1e-6, atol=1e-9)


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_bruteforce_agrees(reduction):
    X, W, Xt, Wt, y = tiny(5, T=4, H=3, Ht=2, V=5, ignore=(3,))
    a = distill_reference(X, W, Xt, Wt, y, temperature=0.8, reduction=reduction)
    b = distill_bruteforce(X, W, Xt, Wt, y, temperature=0.8, reduction=reduction)
    assert a["loss"] == pytest.approx(b["loss"], rel=1e-12)
    np.testing.assert_allclose(a["dX"], np.array(b["dX"]), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(a["dW"], np.array(b["dW"]), rtol=1e-11, atol=1e-14)


def test_ignored_tokens_contribute_nothing():
    X, W, Xt, Wt, y = tiny(6, T=7, ignore=(1, 4))
    ref = distill_reference(X, W, Xt, Wt, y, temperature=1.2)
    assert np.all(ref["dX"][[1, 4]] == 0.0)
    X2, Xt2 = X.copy(), Xt.copy()
    X2[4] += 3.0
    Xt2[1] -= 2.0
    alt = distill_reference(X2, W, Xt2, Wt, y, temperature=1.2)
    assert alt["loss"] == pytest.approx(ref["loss"], rel=1e-13)
    np.testing.assert_allclose(alt["dW"], ref["dW"], rtol=1e-12, atol=1e-15)


def test_sum_is_n_valid_times_mean():
    X, W, Xt, Wt, y = tiny(7, T=9)
    m = distill_reference(X, W, Xt, Wt, y, temperature=1.1, reduction="mean")
    s = distill_reference(X, W, Xt, Wt, y, temperature=1.1, reduction="sum")
    n = int((y != -100).sum())
    assert s["loss"] == pytest.approx(n * m["loss"], rel=1e-12)
    np.testing.assert_allclose(s["dW"], n * m["dW"], rtol=1e-11)


def test_planted_mistakes_are_caught():
    """Each plausible slip in the gradient fails a pin above: a flipped sign
    of (p - q) or a missing 1 / tau breaks the finite differences, a q that
    is not normalised breaks the identical-teacher zero gradient."""
    X, W, Xt, Wt, y = tiny(8, T=5, H=4, Ht=3, V=7, ignore=(1,))
    tau = 1.7
    ref = distill_reference(X, W, Xt, Wt, y, temperature=tau)
    eps = 1e-6
    num = np.zeros_like(W)
    for idx in np.ndindex(W.shape):
        a1 = W.copy(); a1[idx] += eps
        a2 = W.copy(); a2[idx] -= eps
        num[idx] = (distill_reference(X, a1, Xt, Wt, y, temperature=tau, want_grads=False)["loss"]
                    - distill_reference(X, a2, Xt, Wt, y, temperature=tau,
                                        want_grads=False)["loss"]) / (2 * eps)
    for wrong in (-ref["dW"], ref["dW"] * tau):
        assert not np.allclose(num, wrong, rtol=1e-6, atol=1e-9)
    p = softmax((X @ W.T) / tau, axis=1)
    g_unnormalised = (p - 2.0 * p) * ((y != -100) / (y != -100).sum() / tau)[:, None]
    assert np.abs(g_unnormalised.T @ X).max() > 1e-3
