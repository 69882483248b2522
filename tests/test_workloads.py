"""The seeded input recipe: exact ignored-token counts, ignored runs, truncated
Zipf targets, outlier rows of W and round-to-nearest-even bf16 rounding.

The parity tests and the benchmark consume these inputs, so the recipe is
pinned here against what the five configurations fix (ignore shares, run
lengths, the Zipf exponent, the outlier share and scale) and against torch's
own float32 -> bfloat16 conversion.
"""
import numpy as np
import pytest

import workloads


def ignore_mask(n):
    wl = workloads.WORKLOADS[n]
    ss = np.random.SeedSequence(wl.seed).spawn(4)
    rm = np.random.Generator(np.random.PCG64(ss[3]))
    return wl, workloads.ignore_positions(rm, wl.T, wl.ignore_frac, wl.ignore_mode)


# counted tokens T - round(share * T) for the shares the configurations give:
# 10 % of 128, 5 % of 4096 and of 65536, 2 % of 16384, 25 % of 8192
@pytest.mark.parametrize("n,n_valid", [(1, 115), (2, 3891), (3, 62259), (4, 16056), (5, 6144)])
def test_ignored_counts_are_exact(n, n_valid):
    wl, mask = ignore_mask(n)
    assert wl.T - int(mask.sum()) == n_valid


def test_ignored_runs_are_contiguous():
    wl, mask = ignore_mask(5)
    assert wl.ignore_mode == "runs" and int(mask.sum()) == 2048
    edges = np.flatnonzero(np.diff(np.concatenate(([0], mask.astype(np.int8), [0]))))
    starts, ends = edges[::2], edges[1::2]
    # runs of 32 to 512 tokens (the last one cut short), which may touch:
    # at most 2048 / 32 maximal runs, against ~2000 for scattered positions
    assert 1 <= len(starts) <= 2048 // 32
    assert int((ends - starts).sum()) == 2048
    scattered = workloads.ignore_positions(np.random.default_rng(0), wl.T, 0.25, "scatter")
    assert int(np.count_nonzero(np.diff(scattered.astype(np.int8)) == 1)) > 1000


def test_zipf_targets_follow_the_truncated_law():
    V, s, n = 128256, 1.1, 400000
    y = workloads.zipf_targets(np.random.default_rng(7), n, V, s)
    assert y.min() >= 0 and y.max() < V
    p = (np.arange(1, V + 1, dtype=np.float64) ** -s)
    p /= p.sum()
    for k in range(5):
        f = np.count_nonzero(y == k) / n
        sd = np.sqrt(p[k] * (1 - p[k]) / n)
        assert abs(f - p[k]) <= 5 * sd, (k, f, p[k])
    # the tail: ids beyond 10000 carry their share of the mass
    tail = np.count_nonzero(y >= 10000) / n
    assert abs(tail - p[10000:].sum()) <= 5 * np.sqrt(p[10000:].sum() / n)


def test_outlier_rows_of_w():
    wl = workloads.WORKLOADS[5].with_shape(T=64, H=256, V=12800, seed=9)
    inp = workloads.generate(wl)
    norms = np.linalg.norm(inp.W, axis=1)
    big = norms > 5 * np.median(norms)
    assert int(big.sum()) == round(wl.outlier_frac * wl.V) == 13
    assert np.allclose(np.median(norms[big]) / np.median(norms[~big]), wl.outlier_scale, rtol=0.1)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    a = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    # exact halfway cases: low 16 bits 0x8000, both parities of the kept bit
    u = rng.integers(0, 2 ** 31, 2000, dtype=np.uint64).astype(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties)]
    a = np.concatenate([a, ties, np.float32([0.0, -0.0, np.inf, -np.inf])])
    ours = workloads.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = workloads.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_generate_is_deterministic():
    wl = workloads.WORKLOADS[4].with_shape(T=300, H=64, V=5000, seed=11)
    a, b = workloads.generate(wl), workloads.generate(wl)
    assert np.array_equal(a.x_bits, b.x_bits) and np.array_equal(a.w_bits, b.w_bits)
    assert np.array_equal(a.y, b.y)
    c = workloads.generate(wl.with_shape(seed=12))
    assert not np.array_equal(a.x_bits, c.x_bits)
