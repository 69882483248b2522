"""GPU parity: the HIP path through the C ABI vs the float64 oracle.

Sizes here let the full oracle finish in seconds while spanning several
GEMM tiles, several token chunks and ragged tails in every dimension.
"""
import dataclasses

import numpy as np
import pytest

import linear_cross_entropy_02_amd as flce
import workloads
from flce_check import check_full, rel_frob, to_np
from oracle import flce_reference

pytestmark = pytest.mark.gpu


def run(wl, chunk=0, inp=None, out=None, op=None, dw_chunks=0, weight_copy=True):
    import torch
    if inp is None:
        inp = workloads.generate(wl)
    X, W, y = workloads.to_torch(inp, "cuda")
    own = op is None
    if own:
        op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=chunk,
                                          dw_chunks=dw_chunks, weight_copy=weight_copy)
    print(f"[gpu] {wl.name} T={wl.T} H={wl.H} V={wl.V} {wl.dtype} chunk={op.chunk_tokens} "
          f"dw_chunks={op.dw_chunks} weight_copy={weight_copy}", flush=True)
    res = op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction, out=out)
    torch.cuda.synchronize()
    if own:
        op.close()
    return inp, res


def oracle(inp, wl):
    return flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction)


CASES = [
    # (workload, chunk)
    (workloads.WORKLOADS[1], 0),                                            # tiny fp32, full
    (workloads.WORKLOADS[1].with_shape(T=200, V=777, seed=7), 64),          # fp32 ragged, 4 chunks
    (workloads.WORKLOADS[2], 0),                                            # page-1 layer shape, full
    (workloads.WORKLOADS[2].with_shape(T=1000, H=96, V=1000, seed=11), 256),  # ragged T/H/V
    (workloads.WORKLOADS[2].with_shape(T=777, H=264, V=2049, seed=12), 512),  # H % 64 != 0
    (workloads.WORKLOADS[4].with_shape(T=600, H=1024, V=20000, seed=13), 256),  # zipf head
    (workloads.WORKLOADS[5].with_shape(T=700, H=512, V=12345, seed=14), 256),   # outliers, runs, sum
    # dX of a 2048-token chunk at H = 2048 is 64 tiles of 256 x 256: K split
    # four ways over the vocabulary, then the partials summed
    (workloads.WORKLOADS[4].with_shape(T=2100, H=2048, V=16500, seed=15), 2048),
    # the same 64 dX tiles over a 9000-word vocabulary: 35 K-steps per split,
    # the short splits that the 65536 x 512 x 16000 workload runs on
    (workloads.WORKLOADS[4].with_shape(T=2100, H=2048, V=9000, seed=22), 2048),
    # its dW grid (65 x 8 = 520 tiles on 256 CUs) splits the last 8 tiles four
    # ways in K and sums them in a second pass, both when the first chunk
    # stores dW and when the second accumulates into it
    (workloads.WORKLOADS[4].with_shape(T=4200, H=2048, V=16500, seed=18), 2048),
    # an 8192-token chunk at H = 512, V = 16000: its 126 dW tiles (under half
    # a round) split two ways in K as a whole; the 108-token second chunk
    # accumulates through 128-wide tiles
    (workloads.WORKLOADS[3].with_shape(T=8300, seed=23), 8192),
    # 33 x 10 = 330 dW tiles: one full round of 256, then the last 74 split
    # three ways in K, unevenly (32 K-steps as 11/11/10 when the first chunk
    # stores dW, 31 as 11/11/9 when the second, ragged one accumulates)
    (workloads.WORKLOADS[4].with_shape(T=4000, H=2560, V=8300, seed=24), 2048),
    # a 1536-token chunk at H = 4096: 96 dX tiles, split two ways (192 blocks,
    # one round) rather than three (288 blocks, two rounds); the 64-token
    # second chunk takes 128-wide tiles split eight ways
    (workloads.WORKLOADS[4].with_shape(T=1600, H=4096, V=9000, seed=25), 1536),
    # 38 x 16 = 608 dW tiles: the last 96 split two ways
    (workloads.WORKLOADS[4].with_shape(T=4200, H=4096, V=9700, seed=19), 2048),
    # the same split of the dW grid on fp32 operands
    (workloads.WORKLOADS[1].with_shape(T=2100, H=2048, V=16500, seed=21), 2048),
    # a vocabulary of more than 1024 partial tiles: the merge keeps 1024 of
    # them per row block in registers and reads the rest in each pass
    (workloads.WORKLOADS[4].with_shape(T=100, H=64, V=140000, seed=20), 256),
    # degenerate sizes: one K-step shorter than a stage, a vocabulary smaller
    # than one 128-column partial tile
    (workloads.WORKLOADS[2].with_shape(T=300, H=8, V=50, seed=16), 256),
    (workloads.WORKLOADS[1].with_shape(T=70, H=4, V=3, seed=17), 64),
]


@pytest.mark.parametrize("wl,chunk", CASES, ids=[c[0].name for c in CASES])
def test_parity_vs_oracle(wl, chunk):
    inp, out = run(wl, chunk)
    ref = oracle(inp, wl)
    check_full(out, ref, inp, wl)


@pytest.mark.parametrize("n", [1, 2])
def test_parity_as_benchmarked(n):
    # the two small workloads in full, in the launch configuration bench.py
    # times (the large ones: test_gpu_full.py)
    wl = workloads.WORKLOADS[n]
    chunk, g = workloads.launch_config(n)
    inp, out = run(wl, chunk, dw_chunks=g, weight_copy=workloads.weight_copy(n))
    check_full(out, oracle(inp, wl), inp, wl)


# dW over groups of G chunks: full groups, a last group cut short by the
# batch, a ragged last chunk, and G larger than the number of chunks
DW_GROUP_CASES = [
    (workloads.WORKLOADS[2].with_shape(T=1000, H=96, V=1000, seed=31), 256, 2),   # 2 groups, last 2nd ragged
    (workloads.WORKLOADS[2].with_shape(T=1044, H=136, V=3001, seed=32), 256, 2),  # last group = 1 ragged chunk
    (workloads.WORKLOADS[4].with_shape(T=900, H=512, V=20000, seed=33), 256, 3),  # 1 full + 1 partial group
    (workloads.WORKLOADS[1].with_shape(T=200, V=777, seed=34), 64, 8),            # fp32, G > chunks
]


@pytest.mark.parametrize("wl,chunk,g", DW_GROUP_CASES,
                         ids=[f"{c[0].name}-G{c[2]}" for c in DW_GROUP_CASES])
def test_parity_dw_chunk_groups(wl, chunk, g):
    inp, out = run(wl, chunk, dw_chunks=g)
    check_full(out, oracle(inp, wl), inp, wl)


# dX reading W as stored (transposing LDS reads, no W^T copy): 128-wide
# tiles with ragged T/H/V, H % 64 != 0, 256-wide tiles split four ways in K,
# a full 256-wide grid on the outlier-row head, degenerate sizes
NO_WCOPY_CASES = [
    (workloads.WORKLOADS[2].with_shape(T=1000, H=96, V=1000, seed=41), 256),
    (workloads.WORKLOADS[2].with_shape(T=777, H=264, V=2049, seed=42), 512),
    (workloads.WORKLOADS[4].with_shape(T=2100, H=2048, V=9000, seed=43), 2048),
    (workloads.WORKLOADS[5].with_shape(T=2100, H=8192, V=3000, seed=44), 2048),
    (workloads.WORKLOADS[2].with_shape(T=300, H=8, V=50, seed=45), 256),
    # a wide hidden size that is not a multiple of 64 (313 K-steps of the
    # logits GEMM, the last one masked; dW through the dZ pass above H = 4096)
    (workloads.WORKLOADS[4].with_shape(T=300, H=20008, V=3000, seed=49), 256),
]


@pytest.mark.parametrize("wl,chunk", NO_WCOPY_CASES, ids=[c[0].name for c in NO_WCOPY_CASES])
def test_parity_no_weight_copy(wl, chunk):
    import torch
    inp = workloads.generate(wl)
    inp, out = run(wl, chunk, inp=inp, weight_copy=False)
    check_full(out, oracle(inp, wl), inp, wl)
    # the same products in the same order as through the copy: bit for bit
    _, ref = run(wl, chunk, inp=inp)
    for k in ("loss", "dX", "dW", "lse", "argmax", "n_valid"):
        assert torch.equal(out[k], ref[k]), k


def test_vocabulary_at_the_size_limit():
    # the widest vocabulary a handle takes: rows padded to 2^20 columns, 8192
    # partial tiles per row (the merge's uncached tiles, the row-reference
    # pass's eight passes over its shift bytes), 256-row operand tiles of
    # 2^29 bytes at 32-bit offsets, and dW reading two 256-token chunks of
    # exponentials (2^30 bytes under its one buffer descriptor); W through
    # the copy, then as stored, bit for bit
    import torch
    wl = workloads.WORKLOADS[2].with_shape(T=300, H=64, V=(1 << 20) - 300, seed=48)
    inp = workloads.generate(wl)
    inp, out = run(wl, 256, inp=inp, dw_chunks=2)
    ref = flce_reference(inp.X, inp.W, inp.y, wl.ignore_index, wl.reduction, chunk=64)
    check_full(out, ref, inp, wl)
    del ref
    _, out2 = run(wl, 256, inp=inp, dw_chunks=2, weight_copy=False)
    for k in ("loss", "dX", "dW", "lse", "argmax", "n_valid"):
        assert torch.equal(out[k], out2[k]), k


def test_no_weight_copy_workspace_and_dtype():
    wl = workloads.WORKLOADS[2].with_shape(T=300, H=256, V=3000, seed=46)
    a = flce.FusedLinearCrossEntropy(wl.H, wl.V, "bf16", chunk_tokens=256)
    b = flce.FusedLinearCrossEntropy(wl.H, wl.V, "bf16", chunk_tokens=256, weight_copy=False)
    vpad = -(-wl.V // 256) * 256
    assert a.workspace_bytes - b.workspace_bytes == wl.H * vpad * 2
    a.close()
    b.close()
    with pytest.raises(flce.FlceError):
        flce.FusedLinearCrossEntropy(64, 300, "f32", weight_copy=False)


def test_all_tokens_ignored():
    wl = workloads.WORKLOADS[2].with_shape(T=300, H=128, V=1000, seed=21)
    inp = workloads.generate(wl)
    inp.y[:] = wl.ignore_index
    inp, out = run(wl, 0, inp=inp)
    assert float(out["loss"].item()) == 0.0
    assert int(out["n_valid"].item()) == 0
    assert np.all(to_np(out["dX"]) == 0.0)
    assert np.all(to_np(out["dW"]) == 0.0)
    ref = oracle(inp, wl)
    assert np.abs(to_np(out["lse"]) - ref["lse"]).max() <= 1e-3


@pytest.mark.parametrize("reduction", ["mean", "sum"])
def test_none_ignored_and_vocab_ends(reduction):
    import dataclasses
    wl = dataclasses.replace(workloads.WORKLOADS[2].with_shape(T=500, H=128, V=3000, seed=22),
                             ignore_frac=0.0, reduction=reduction)
    inp = workloads.generate(wl)
    inp.y[::2] = 0
    inp.y[1::2] = wl.V - 1
    inp, out = run(wl, 128, inp=inp)
    check_full(out, oracle(inp, wl), inp, wl)


def test_ignore_index_is_a_real_vocab_id():
    import dataclasses
    wl = dataclasses.replace(workloads.WORKLOADS[2].with_shape(T=400, H=64, V=500, seed=23),
                             ignore_index=7, ignore_frac=0.0)
    inp = workloads.generate(wl)
    inp.y[::5] = 7
    inp, out = run(wl, 0, inp=inp)
    check_full(out, oracle(inp, wl), inp, wl)


def test_empty_batch():
    import torch
    wl = workloads.WORKLOADS[2].with_shape(T=0, H=64, V=300, seed=24)
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, "bf16")
    W = torch.randn(wl.V, wl.H, device="cuda").to(torch.bfloat16)
    out = op.alloc_outputs(0, "cuda")
    out["dW"].fill_(1.0)
    st = flce.flce_fwd_bwd(op.handle, None, W, None, 0, -100, flce.FLCE_MEAN, out["loss"], None,
                           out["dW"], None, None, out["n_valid"])
    assert st == flce.FLCE_OK
    torch.cuda.synchronize()
    assert float(out["loss"].item()) == 0.0
    assert int(out["n_valid"].item()) == 0
    assert torch.all(out["dW"] == 0).item()
    op.close()


def test_out_of_range_targets_are_counted_and_ignored():
    wl = workloads.WORKLOADS[2].with_shape(T=256, H=64, V=400, seed=25)
    inp = workloads.generate(wl)
    y_bad = inp.y.copy()
    y_bad[[3, 50, 51]] = [wl.V, -5, 10 ** 9]
    inp_bad = workloads.Inputs(wl, inp.X, inp.W, y_bad, inp.x_bits, inp.w_bits)
    import torch
    X, W, y = workloads.to_torch(inp_bad, "cuda")
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, "bf16")
    out = op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction)
    st, bad = flce.flce_query_error(op.handle)
    assert st == flce.FLCE_ERR_BAD_TARGET and bad == 3
    y_ref = y_bad.copy()
    y_ref[[3, 50, 51]] = wl.ignore_index
    inp_ref = workloads.Inputs(wl, inp.X, inp.W, y_ref, inp.x_bits, inp.w_bits)
    check_full(out, oracle(inp_ref, wl), inp_ref, wl)
    # a clean call resets the count
    out = op.fwd_bwd(*workloads.to_torch(inp, "cuda"), wl.ignore_index, wl.reduction)
    st, bad = flce.flce_query_error(op.handle)
    assert st == flce.FLCE_OK and bad == 0
    op.close()


@pytest.mark.parametrize("T", [32767, 40000, 700000])
def test_target_counts_of_long_batches(T):
    # from 32768 targets on, blocks count slices of the batch and a second
    # pass sums them: n_valid and the out-of-range count stay exact
    import dataclasses
    import torch
    wl = dataclasses.replace(workloads.WORKLOADS[2].with_shape(T=T, H=8, V=50, seed=26),
                             ignore_frac=0.3)
    inp = workloads.generate(wl)
    y_bad = inp.y.copy()
    bad_rows = np.random.default_rng(5).choice(T, size=37, replace=False)
    y_bad[bad_rows] = wl.V + 3
    X, W, _ = workloads.to_torch(inp, "cuda")
    y = torch.from_numpy(y_bad).to("cuda")
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, "bf16", chunk_tokens=8192)
    out = op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction)
    st, bad = flce.flce_query_error(op.handle)
    assert st == flce.FLCE_ERR_BAD_TARGET and bad == 37
    valid = (y_bad != wl.ignore_index) & (y_bad >= 0) & (y_bad < wl.V)
    assert int(out["n_valid"].item()) == int(valid.sum())
    op.close()


def test_bad_arguments_rejected_without_work():
    import torch
    op = flce.FusedLinearCrossEntropy(64, 300, "bf16")
    X = torch.zeros(10, 64, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(300, 64, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(10, dtype=torch.int64, device="cuda")
    out = op.alloc_outputs(10, "cuda")
    h = op.handle
    call = lambda **kw: flce.flce_fwd_bwd(h, kw.get("X", X), kw.get("W", W), kw.get("y", y),
                                          kw.get("T", 10), -100, kw.get("red", flce.FLCE_MEAN),
                                          kw.get("loss", out["loss"]), kw.get("dX", out["dX"]),
                                          kw.get("dW", out["dW"]))
    E = flce.FLCE_ERR_INVALID_ARGUMENT
    assert call(T=-1) == E
    assert call(red=0) == E
    assert call(red=3) == E
    assert call(X=0) == E
    assert call(W=0) == E
    assert call(y=0) == E
    assert call(loss=0) == E
    assert call(dX=0) == E
    assert call(dW=0) == E
    assert call(X=X.data_ptr() + 2) == E          # misaligned
    assert call() == flce.FLCE_OK
    torch.cuda.synchronize()
    op.close()


def test_deterministic_bitwise():
    wl = workloads.WORKLOADS[2].with_shape(T=1500, H=256, V=5000, seed=26)
    inp = workloads.generate(wl)
    _, a = run(wl, 512, inp=inp)
    _, b = run(wl, 512, inp=inp)
    for k in ("loss", "dX", "dW", "lse", "argmax"):
        assert np.array_equal(to_np(a[k]), to_np(b[k])), k


def test_chunk_size_invariance():
    wl = workloads.WORKLOADS[4].with_shape(T=1100, H=256, V=7000, seed=27)
    inp = workloads.generate(wl)
    outs = [run(wl, c, inp=inp)[1] for c in (256, 512, 2048)]
    ref = oracle(inp, wl)
    for o in outs:
        check_full(o, ref, inp, wl)
    assert rel_frob(to_np(outs[0]["dW"]), to_np(outs[2]["dW"])) < 1e-2


def test_workspace_does_not_depend_on_tokens():
    """The workspace is sized at create time from (H, V, C) only; the part
    that holds logit-shaped chunk buffers is C x V, below T x V."""
    op = flce.FusedLinearCrossEntropy(512, 16000, "bf16", chunk_tokens=1024)
    ws = op.workspace_bytes
    wl = workloads.WORKLOADS[2]
    for T in (1024, 4096):
        inp = workloads.generate(wl.with_shape(T=T))
        run(wl.with_shape(T=T), inp=inp, op=op)
        assert op.workspace_bytes == ws
    assert ws < 4096 * 16000 * 2
    op.close()


def test_non_finite_inputs_poison_like_the_oracle():
    # A NaN row of W makes every logit of that vocabulary id NaN, so every
    # token's lse, the loss and the gradients are NaN; a +inf entry of X
    # makes that token's logits infinite (NaN after the max is subtracted):
    # its lse and the loss are NaN while every other token's lse stays
    # finite and exact.  The oracle is the reference for which is which.
    import torch
    wl = workloads.WORKLOADS[2].with_shape(T=300, H=128, V=1500, seed=27)
    base = workloads.generate(wl)
    first_valid = int(np.nonzero(base.y != wl.ignore_index)[0][0])
    cases = {"nan_w_row": ("W", 5, None), "inf_x": ("X", first_valid, 7)}
    for name, (which, r, c) in cases.items():
        X = base.X.copy()
        W = base.W.copy()
        if which == "W":
            W[r, :] = np.nan
        else:
            X[r, c] = np.inf
        inp = workloads.Inputs(wl, X, W, base.y, workloads.f32_to_bf16_bits(X),
                               workloads.f32_to_bf16_bits(W))
        print(f"[gpu] non-finite case {name}", flush=True)
        _, out = run(wl, 256, inp=inp)
        with np.errstate(invalid="ignore", over="ignore"):
            ref = oracle(inp, wl)
        lse = to_np(out["lse"])
        assert np.isnan(float(out["loss"].item())) == np.isnan(ref["loss"]), name
        assert np.array_equal(np.isnan(lse), np.isnan(ref["lse"])), name
        fin = ~np.isnan(ref["lse"])
        if fin.any():
            assert np.abs(lse[fin] - ref["lse"][fin]).max() <= 1e-3, name
        assert np.isnan(ref["loss"]), name


# Degenerate heads: one token; every token ignored (the mean over zero
# tokens is defined as 0, and so are its gradients); one valid token among
# ignored ones; a sum over a batch with a single valid token
DEGENERATE_CASES = [
    dataclasses.replace(workloads.WORKLOADS[2].with_shape(T=1, H=64, V=1000, seed=51),
                        ignore_frac=0.0),
    dataclasses.replace(workloads.WORKLOADS[2].with_shape(T=300, H=64, V=700, seed=52),
                        ignore_frac=1.0),
    dataclasses.replace(workloads.WORKLOADS[2].with_shape(T=300, H=64, V=700, seed=53),
                        ignore_frac=1.0, reduction="sum"),
    dataclasses.replace(workloads.WORKLOADS[1].with_shape(T=1, H=16, V=40, seed=54),
                        ignore_frac=0.0),
]


@pytest.mark.parametrize("wl", DEGENERATE_CASES,
                         ids=[f"{c.name}-T{c.T}-ign{c.ignore_frac}-{c.reduction}"
                              for c in DEGENERATE_CASES])
def test_degenerate_heads(wl):
    inp, out = run(wl, 256)
    ref = oracle(inp, wl)
    check_full(out, ref, inp, wl)
    if wl.ignore_frac == 1.0:
        assert ref["n_valid"] == 0
        assert float(out["loss"].item()) == 0.0
        assert not to_np(out["dX"]).any() and not to_np(out["dW"]).any()


def test_single_valid_token_among_ignored():
    wl = dataclasses.replace(workloads.WORKLOADS[2].with_shape(T=500, H=128, V=3000, seed=55),
                             ignore_frac=0.0)
    inp = workloads.generate(wl)
    inp.y[:] = wl.ignore_index
    inp.y[317] = 1234
    inp, out = run(wl, 256, inp=inp)
    ref = oracle(inp, wl)
    assert ref["n_valid"] == 1
    check_full(out, ref, inp, wl)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_word_vocabulary(dtype):
    # V = 1: the softmax is 1, so loss and gradients vanish up to the rounding
    # of lse - z; lse equals the single logit and the argmax is 0
    base = workloads.WORKLOADS[2] if dtype == "bf16" else workloads.WORKLOADS[1]
    wl = dataclasses.replace(base.with_shape(T=700, H=64, V=1, seed=56), ignore_frac=0.1)
    inp, out = run(wl, 256)
    ref = oracle(inp, wl)
    z = inp.X.astype(np.float64) @ inp.W.astype(np.float64).T
    lse = to_np(out["lse"])
    assert np.abs(lse - z[:, 0]).max() <= 1e-5 * max(1.0, np.abs(z).max())
    assert np.all(to_np(out["argmax"]) == 0)
    assert int(out["n_valid"].item()) == ref["n_valid"]
    assert abs(float(out["loss"].item())) <= 1e-6
    # |dX_t| = s |p - 1| |W_0| with |p - 1| at the rounding of exp(z - lse)
    s = 1.0 / ref["n_valid"]
    wn = float(np.linalg.norm(inp.W.astype(np.float64)))
    assert np.linalg.norm(to_np(out["dX"]), axis=1).max() <= 1e-5 * s * wn
    assert np.linalg.norm(to_np(out["dW"])) <= 1e-5 * np.linalg.norm(inp.X.astype(np.float64))
