"""GPU parity of the two ways dZ reaches the dX contraction, against the
oracle.

Default: the dX and dW contractions read the stored exponentials and form
dZ themselves.  Their tile references are powers 2^(32 j); the row-reference
pass rewrites in place the row segments whose reference lies below their
row's (so that each row's exponentials share one) and sets the target column;
each output row of dX is finished with the row's scale plus the target's
correction times that row of W, and dW contracts the exponentials as stored
against the row-scaled X^T (bf16 up to H = 4096; elsewhere the dZ pass writes
dZ^T for it).  FLCE_FLAG_DZ_IN_PLACE: the dZ pass writes dZ over the
exponentials and dZ^T, and the contractions read those.

The rest of the GPU suite runs the default; the cases here run the in-place
mode over every instantiation both paths have (256-wide tiles split in K and
written directly, 128-wide tiles split and direct, fp32, W read as stored,
several chunks with dW groups, the outlier-row head with its wide logit
range, ignored runs, targets at both vocabulary ends, an ignore index that is
a real id, a vocabulary shard's backward), compare the two modes, and give
the default rows whose tiles straddle a reference.
"""
import dataclasses

import numpy as np
import pytest

import linear_cross_entropy_02_amd as flce
import workloads
from flce_check import check_full, rel_frob, to_np
from oracle import flce_reference

pytestmark = pytest.mark.gpu


def run(wl, chunk, dw_chunks=0, weight_copy=True, dz_in_place=True, inp=None):
    import torch
    if inp is None:
        inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=chunk,
                                      dw_chunks=dw_chunks, weight_copy=weight_copy,
                                      dz_in_place=dz_in_place)
    print(f"[gpu-dz-modes] {wl.name} T={wl.T} H={wl.H} V={wl.V} {wl.dtype} chunk={op.chunk_tokens} "
          f"G={op.dw_chunks} wcopy={weight_copy} dz_in_place={dz_in_place}", flush=True)
    out = op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction)
    torch.cuda.synchronize()
    op.close()
    return inp, out


CASES = [
    # (workload, chunk, dW chunks, W^T copy)
    (workloads.WORKLOADS[2], 1024, 1, True),             # 128-wide tiles, K split 8 ways
    (workloads.WORKLOADS[4].with_shape(T=2100, H=2048, V=16500, seed=71), 2048, 1, True),  # 256, split 4
    (workloads.WORKLOADS[4].with_shape(T=5000, H=4096, V=3000, seed=72), 4096, 1, True),   # 256, direct
    (workloads.WORKLOADS[2].with_shape(T=700, H=256, V=300, seed=73), 256, 1, True),       # 128, direct
    (workloads.WORKLOADS[1], 0, 1, True),                # fp32
    (workloads.WORKLOADS[1].with_shape(T=200, V=777, seed=74), 64, 2, True),  # fp32, 4 chunks, G = 2
    (workloads.WORKLOADS[4].with_shape(T=2100, H=2048, V=9000, seed=75), 2048, 1, False),  # W as stored
    (workloads.WORKLOADS[2].with_shape(T=777, H=264, V=2049, seed=76), 512, 1, False),
    (workloads.WORKLOADS[5].with_shape(T=700, H=512, V=12345, seed=77), 256, 1, True),     # outliers
    (workloads.WORKLOADS[5].with_shape(T=2100, H=8192, V=3000, seed=78), 2048, 1, False),
    (workloads.WORKLOADS[2].with_shape(T=1000, H=96, V=1000, seed=79), 256, 2, True),      # G groups
]


@pytest.mark.parametrize("wl,chunk,g,wcopy", CASES,
                         ids=[f"{c[0].name}-C{c[1]}-G{c[2]}" + ("" if c[3] else "-no-wcopy")
                              for c in CASES])
def test_dz_in_place_vs_oracle(wl, chunk, g, wcopy):
    inp, out = run(wl, chunk, g, wcopy)
    ref = flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction)
    check_full(out, ref, inp, wl)


def test_the_two_modes_agree():
    # the same gradients up to bf16 rounding of dZ (formed in registers
    # against written out); lse, argmax, counts and the loss come from the
    # same kernels and are identical
    wl = workloads.WORKLOADS[4].with_shape(T=1500, H=512, V=20000, seed=80)
    inp = workloads.generate(wl)
    _, a = run(wl, 512, inp=inp)
    _, b = run(wl, 512, inp=inp, dz_in_place=False)
    for k in ("loss", "lse", "argmax", "n_valid"):
        assert np.array_equal(to_np(a[k]), to_np(b[k])), k
    assert rel_frob(to_np(a["dX"]), to_np(b["dX"])) < 1e-2
    assert rel_frob(to_np(a["dW"]), to_np(b["dW"])) < 1e-2


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_dz_in_place_targets_at_vocab_ends_and_real_ignore_id(reduction):
    wl = dataclasses.replace(workloads.WORKLOADS[2].with_shape(T=600, H=128, V=3000, seed=81),
                             ignore_index=7, ignore_frac=0.0, reduction=reduction)
    inp = workloads.generate(wl)
    inp.y[::3] = 0
    inp.y[1::3] = wl.V - 1
    inp.y[::7] = 7
    inp, out = run(wl, 256, inp=inp)
    check_full(out, flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction), inp, wl)


@pytest.mark.parametrize("dz_in_place", [True, False])
def test_vocab_shard_backward(dz_in_place):
    # a shard's backward from a given lse: the row scale comes from that lse
    import torch
    wl = workloads.WORKLOADS[4].with_shape(T=600, H=512, V=20000, seed=82)
    inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    ref = flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction)
    lse = torch.tensor(ref["lse"], dtype=torch.float32, device="cuda")
    dX = np.zeros((wl.T, wl.H))
    dW = np.zeros((wl.V, wl.H))
    bounds = [0, 7000, 13001, wl.V]
    for v0, v1 in zip(bounds[:-1], bounds[1:]):
        op = flce.FusedLinearCrossEntropy(wl.H, v1 - v0, wl.dtype, chunk_tokens=256,
                                          dz_in_place=dz_in_place)
        Ws = W[v0:v1].contiguous()
        dXp, dWs = op.shard_backward(X, Ws, y, lse, v0, wl.V, wl.ignore_index, wl.reduction)
        torch.cuda.synchronize()
        dX += to_np(dXp)
        dW[v0:v1] = to_np(dWs)
        op.close()
    assert rel_frob(dX, ref["dX"]) <= 2e-2
    assert rel_frob(dW, ref["dW"]) <= 2e-2
    assert np.all(dX[inp.y == wl.ignore_index] == 0.0)


def straddle_inputs(dtype, seed, T=640, V=1024):
    """A head whose vocabulary tiles sit at logit levels around 32 ln 2 (a
    multiple of the 2^32 reference quantum), so that the rows hold tiles on
    both sides of it with comparable softmax mass, plus far tiles: per-row
    references differ and the row-reference pass must rescale.  The eight
    levels repeat over the tiles of a longer vocabulary; the last tile is a
    low one."""
    H = 64
    rng = np.random.default_rng(seed)
    levels = np.array([21.4, 21.7, 22.0, 22.3, 22.6, 21.1, -8.0, 4.0])   # tiles of 128
    nt = -(-V // 128)
    tile_level = levels[np.arange(nt) % len(levels)]
    tile_level[-1] = 4.0
    X = (0.02 * rng.standard_normal((T, H))).astype(np.float32)
    # The levels come from a large first column of X times a small one of W:
    # a tile's common component of W then stays small against W's own rows,
    # so dX does not hinge on cancelling it (bf16 dZ rounds at 2^-9).  The
    # targets lie in the last, low tile, so that no dW row subtracts its
    # target count from a similar softmax mass either.
    X[:, 0] = 1000.0 * (1.0 + 0.02 * rng.standard_normal(T))
    W = (0.02 * rng.standard_normal((V, H))).astype(np.float32)
    W[:, 0] = (np.repeat(tile_level, 128)[:V] + 0.3 * rng.standard_normal(V)) / 1000.0
    y = rng.integers(128 * (nt - 1), V, size=T)
    y[::9] = -100
    base = workloads.WORKLOADS[2] if dtype == "bf16" else workloads.WORKLOADS[1]
    wl = dataclasses.replace(base.with_shape(T=T, H=H, V=V, seed=seed), ignore_index=-100)
    if dtype == "bf16":
        xb, wb = workloads.f32_to_bf16_bits(X), workloads.f32_to_bf16_bits(W)
        inp = workloads.Inputs(wl, workloads.bf16_bits_to_f32(xb), workloads.bf16_bits_to_f32(wb),
                               y, xb, wb)
    else:
        inp = workloads.Inputs(wl, X, W, y)
    return wl, inp


@pytest.mark.parametrize("dtype,T,V", [("bf16", 640, 1024), ("f32", 640, 1024),
                                       # rows of 1563 tiles: the row-reference pass
                                       # reads their shift bytes in two passes of
                                       # up to 1024 tiles
                                       ("bf16", 320, 200003), ("f32", 320, 200003)])
def test_rows_whose_tiles_straddle_a_reference(dtype, T, V):
    wl, inp = straddle_inputs(dtype, 83, T, V)
    # on the host: the tile references q ceil(max log2 e / q), q = 32, differ
    # within a good share of the rows
    nt = -(-V // 128)
    z = np.full((T, 128 * nt), -np.inf)
    z[:, :V] = inp.X.astype(np.float64) @ inp.W.astype(np.float64).T
    kq = np.ceil(z.reshape(T, nt, 128).max(axis=2) * np.log2(np.e) / 32) * 32
    below = kq < kq.max(axis=1, keepdims=True)
    mixed = below.any(axis=1)
    assert mixed.mean() > 0.3, mixed.mean()
    if nt > 1024:
        assert below[:, 1024:].any(axis=1).mean() > 0.3
    # the tiles on either side of the boundary carry comparable mass
    p = np.exp(z - z.max(axis=1, keepdims=True))
    tile_mass = p.reshape(T, nt, 128).sum(axis=2)
    low = np.where(below, tile_mass, 0).sum(axis=1)
    assert np.median(low[mixed] / tile_mass[mixed].sum(axis=1)) > 0.1
    del z, p
    _, out = run(wl, 256, inp=inp, dz_in_place=False)
    check_full(out, flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction), inp, wl)
