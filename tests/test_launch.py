"""The shape-based launch policy (CPU only): it reproduces the settings the
benchmark times for each workload, never chunks beyond the batch, and
keeps fp32 on the W^T copy (reading W as stored is bf16 only)."""
import pytest

import workloads
from linear_cross_entropy_02_amd.launch import suggest_launch


@pytest.mark.parametrize("n", sorted(workloads.WORKLOADS))
def test_policy_matches_the_benchmarked_settings(n):
    wl = workloads.WORKLOADS[n]
    C, G, wcopy = suggest_launch(wl.T, wl.H, wl.V, wl.dtype)
    assert (C, G) == workloads.launch_config(n)
    assert wcopy == workloads.weight_copy(n)


@pytest.mark.parametrize("T,H,V,dtype", [(1, 4096, 128256, "bf16"), (300, 512, 16000, "bf16"),
                                         (5000, 8192, 1000, "bf16"), (70000, 64, 50, "f32"),
                                         (0, 1024, 3000, "bf16")])
def test_policy_bounds(T, H, V, dtype):
    C, G, wcopy = suggest_launch(T, H, V, dtype)
    assert C % 256 == 0 and 256 <= C <= max(256, -(-T // 256) * 256)
    assert 1 <= G <= max(1, -(-T // C))
    assert wcopy or dtype == "bf16"
