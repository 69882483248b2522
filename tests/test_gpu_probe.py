"""The MFMA throughput probe on the GPU does the work it is credited with.

Zero operands leave every sum at zero.  With random operands, each wave's
total (the sum of its 64 lanes' sink values) equals iters times the sum of
all elements of its products A_f.B_g, which a host model gets without the
output layout: the sum of all elements of A.B is sum_k (column sum of A at
k) * (row sum of B at k), and on both instruction shapes lane l holds, as
its j-th bf16 of either operand, the k index 8*(l // (64 / (K / 8))) + j
(K = 32 for 16x16x32, 16 for 32x32x16), A's row or B's column being the
rest of l.  The host rebuilds every lane's operands from the probe's
counter-based generator (its hash and bf16 packing restated here)."""
import numpy as np
import pytest

from linear_cross_entropy_02_amd import probe

pytestmark = pytest.mark.gpu
M32 = 0xFFFFFFFF


def mix(x):
    x &= M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & M32
    x ^= x >> 16
    return x


def bf16_pair(h):
    lo = ((h & 0x807F) | ((119 + ((h >> 8) & 15)) << 7)) & 0xFFFF
    g = mix(h)
    hi = ((g & 0x807F) | ((119 + ((g >> 8) & 15)) << 7)) & 0xFFFF
    return lo, hi


def bf16_value(bits):
    return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])


def lane_fragments(tid):
    """A and B fragments (4 each, 8 bf16 values) of global thread `tid`."""
    seed = (tid * 0x9E3779B9) & M32
    a = np.zeros((4, 8))
    b = np.zeros((4, 8))
    for f in range(4):
        for r in range(4):
            for dst, off in ((a, 0), (b, 4)):
                lo, hi = bf16_pair(mix(seed + 8 * f + r + off))
                dst[f, 2 * r] = bf16_value(lo)
                dst[f, 2 * r + 1] = bf16_value(hi)
    return a, b


def wave_expectation(shape, first_tid):
    groups = 4 if shape == 16 else 2          # lanes sharing one k block of 8
    per = 64 // groups
    frags = [lane_fragments(first_tid + l) for l in range(64)]
    A = np.stack([f[0] for f in frags])       # [lane, fragment, j]
    B = np.stack([f[1] for f in frags])
    SA = A.reshape(groups, per, 4, 8).sum(axis=1)   # [k block, fragment, j]
    SB = B.reshape(groups, per, 4, 8).sum(axis=1)
    AA = np.abs(A).reshape(groups, per, 4, 8).sum(axis=1)
    AB = np.abs(B).reshape(groups, per, 4, 8).sum(axis=1)
    pairs = ([(k & 3, (k >> 2) & 3) for k in range(16)] if shape == 16 else
             [(k & 3, (k >> 1) & 3) for k in range(8)])
    total = sum(float((SA[:, fa] * SB[:, fb]).sum()) for fa, fb in pairs)
    scale = sum(float((AA[:, fa] * AB[:, fb]).sum()) for fa, fb in pairs)
    return total, scale


@pytest.mark.parametrize("shape", [16, 32])
def test_probe_sums(shape):
    import torch
    blocks, iters = 2, 3
    print(f"[gpu-probe] shape={shape} blocks={blocks} iters={iters}", flush=True)
    sink = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    probe.mfma_stream(shape, blocks, iters, False, sink)
    torch.cuda.synchronize()
    assert bool((sink == 0).all())
    sink.fill_(float("nan"))
    probe.mfma_stream(shape, blocks, iters, True, sink)
    torch.cuda.synchronize()
    got = sink.double().cpu().numpy().reshape(blocks * 4, 64).sum(axis=1)
    for w in range(blocks * 4):
        want, scale = wave_expectation(shape, 64 * w)
        assert abs(got[w] - iters * want) <= 1e-4 * iters * scale, (w, got[w], iters * want)
