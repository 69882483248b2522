"""The allocation-free entry point (flce_fwd_bwd_noalloc) against flce_fwd_bwd.

It runs the same kernels in the same order on a workspace bound to the
library's static device scratch, so its outputs must equal those of a handle
made with the same configuration, bit for bit -- on two calls in a row, the
second with fewer tokens (the scratch keeps the first call's contents).  A
configuration whose workspace exceeds the scratch is refused with nothing
enqueued, and no call after the first on a device takes device memory.
"""
import numpy as np
import pytest

import linear_cross_entropy_02_amd as flce
import workloads

pytestmark = pytest.mark.gpu

KEYS = ("loss", "dX", "dW", "lse", "argmax", "n_valid")


def noalloc_call(wl, X, W, y, out, chunk, dw_chunks=0, flags=0):
    dt = flce.FLCE_BF16 if wl.dtype == "bf16" else flce.FLCE_F32
    red = flce.FLCE_MEAN if wl.reduction == "mean" else flce.FLCE_SUM
    return flce.flce_fwd_bwd_noalloc(wl.H, wl.V, dt, X, W, y, X.shape[0], wl.ignore_index, red,
                                     out["loss"], out["dX"], out["dW"], out["lse"],
                                     out["argmax"], out["n_valid"], chunk_tokens=chunk,
                                     dw_chunks=dw_chunks, flags=flags)


@pytest.mark.parametrize("wl,chunk,dwc,wcopy,in_place", [
    (workloads.WORKLOADS[2], 1024, 1, True, False),                          # 4096 x 512 x 16000
    (workloads.WORKLOADS[5].with_shape(T=3000, H=1024, V=9000, seed=61), 1024, 2, False, False),
    (workloads.WORKLOADS[1].with_shape(T=600, H=256, V=3000, seed=62), 256, 1, True, False),
    # dZ written in place, which dW reads as stored (G chunks of it)
    (workloads.WORKLOADS[4].with_shape(T=2000, H=512, V=8000, seed=63), 512, 2, True, True),
], ids=["layer-shape", "outlier-head-no-wcopy-G2", "fp32", "dz-in-place-G2"])
def test_noalloc_equals_handle_on_two_calls(wl, chunk, dwc, wcopy, in_place):
    import torch
    flags = (0 if wcopy else flce.FLCE_FLAG_NO_WEIGHT_COPY) | \
        (flce.FLCE_FLAG_DZ_IN_PLACE if in_place else 0)
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=chunk, dw_chunks=dwc,
                                      weight_copy=wcopy, dz_in_place=in_place)
    assert op.workspace_bytes <= flce.FLCE_NOALLOC_SCRATCH_BYTES
    for k, T in enumerate((wl.T, wl.T // 3 + 5)):
        w = wl.with_shape(T=T, seed=wl.seed + 100 * k)
        inp = workloads.generate(w, keep_f32=False)
        X, W, y = workloads.to_torch(inp, "cuda")
        print(f"[gpu-noalloc] {w.name} call {k}: T={T} H={w.H} V={w.V} chunk={chunk} G={dwc} "
              f"wcopy={wcopy} in_place={in_place}", flush=True)
        ref = op.fwd_bwd(X, W, y, w.ignore_index, w.reduction)
        out = op.alloc_outputs(T, "cuda")
        for t in out.values():
            t.fill_(7)                        # nothing may survive from the fill
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        st = noalloc_call(w, X, W, y, out, chunk, dwc, flags)
        assert st == flce.FLCE_OK, flce.last_error()
        torch.cuda.synchronize()
        if k > 0:
            assert torch.cuda.mem_get_info()[0] == free0, "the call took device memory"
        for key in KEYS:
            assert torch.equal(out[key], ref[key]), key
        assert np.isfinite(float(out["loss"].item()))
    op.close()


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    import torch
    wl = workloads.WORKLOADS[2].with_shape(T=64, H=4096, V=128256, seed=63)
    X = torch.zeros(64, wl.H, dtype=torch.bfloat16, device="cuda")
    W = torch.zeros(wl.V, wl.H, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(64, dtype=torch.int64, device="cuda")
    out = dict(loss=torch.full((), 3.0, device="cuda"),
               dX=torch.full((64, wl.H), 3.0, dtype=torch.bfloat16, device="cuda"),
               dW=torch.full((16, 16), 3.0, device="cuda"), lse=None, argmax=None, n_valid=None)
    st = flce.flce_fwd_bwd_noalloc(wl.H, wl.V, flce.FLCE_BF16, X, W, y, 64, -100, flce.FLCE_MEAN,
                                   out["loss"], out["dX"], out["dW"], chunk_tokens=2048)
    assert st == flce.FLCE_ERR_UNSUPPORTED
    assert "static scratch" in flce.last_error()
    torch.cuda.synchronize()
    assert float(out["loss"].item()) == 3.0     # nothing enqueued
    # bad arguments are refused as by flce_fwd_bwd
    st = flce.flce_fwd_bwd_noalloc(512, 1000, flce.FLCE_BF16, X[:, :512], None, y, 64, -100,
                                   flce.FLCE_MEAN, out["loss"], out["dX"], out["dW"])
    assert st == flce.FLCE_ERR_INVALID_ARGUMENT


def test_noalloc_call_captured_in_a_graph():
    # what the entry point is for: a capturable call with nothing to allocate.
    # The first call on the device (eager) looks the scratch up; the graph's
    # replays, with eager calls on the same scratch between them, must match
    # a handle's results bit for bit.
    import torch
    wl = workloads.WORKLOADS[2].with_shape(T=900, H=256, V=3000, seed=64)
    ins = [workloads.generate(wl.with_shape(seed=64 + k), keep_f32=False) for k in range(2)]
    tens = [workloads.to_torch(i, "cuda") for i in ins]
    op = flce.FusedLinearCrossEntropy(wl.H, wl.V, wl.dtype, chunk_tokens=256, dw_chunks=2)
    refs = [op.fwd_bwd(X, W, y, wl.ignore_index, wl.reduction) for X, W, y in tens]
    Xg, Wg, yg = (t.clone() for t in tens[0])
    out = op.alloc_outputs(wl.T, "cuda")
    print(f"[gpu-noalloc] graph capture {wl.name}", flush=True)
    assert noalloc_call(wl, Xg, Wg, yg, out, 256, 2) == flce.FLCE_OK   # eager, first on device
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = noalloc_call(wl, Xg, Wg, yg, out, 256, 2)
    assert st == flce.FLCE_OK
    torch.cuda.synchronize()
    other = op.alloc_outputs(wl.T, "cuda")
    for r in range(4):
        k = r % 2
        for dst, src in zip((Xg, Wg, yg), tens[k]):
            dst.copy_(src)
        for t in out.values():
            t.zero_()
        g.replay()
        # eager work on the same scratch between replays, in stream order
        assert noalloc_call(wl, *tens[1 - k], other, 256, 2) == flce.FLCE_OK
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(out[key], refs[k][key]), (r, key)
            assert torch.equal(other[key], refs[1 - k][key]), (r, key)
    del g
    op.close()
    assert torch.cuda.mem_get_info()[0] >= free0 - (64 << 20)   # graph bookkeeping only
