"""The seeded generator: determinism, independence of streams, distributions, MoE layout."""
import numpy as np
import torch

import workloads


def test_counter_based_slices_agree():
    full = workloads.normal_f32(3, 77, (1000,))
    part = workloads.normal_f32(3, 77, (300,), first=500)
    assert np.array_equal(full[500:800], part)


def test_deterministic_and_distinct_streams():
    a = workloads.normal_f32(3, workloads.tensor_id(workloads.KIND_PARTIAL, 0), (4096,))
    b = workloads.normal_f32(3, workloads.tensor_id(workloads.KIND_PARTIAL, 0), (4096,))
    c = workloads.normal_f32(3, workloads.tensor_id(workloads.KIND_PARTIAL, 1), (4096,))
    d = workloads.normal_f32(4, workloads.tensor_id(workloads.KIND_PARTIAL, 0), (4096,))
    assert np.array_equal(a, b)
    assert abs(np.corrcoef(a, c)[0, 1]) < 0.05 and abs(np.corrcoef(a, d)[0, 1]) < 0.05


def test_normal_moments():
    v = workloads.normal_f32(9, 1, (400000,), mean=1.0, std=0.1).astype(np.float64)
    assert abs(v.mean() - 1.0) < 1e-3 and abs(v.std() - 0.1) < 1e-3
    u = workloads.uniform_f64(9, 2, (400000,))
    assert u.min() >= 0.0 and u.max() < 1.0 and abs(u.mean() - 0.5) < 3e-3


def test_outlier_fraction():
    n = 2_000_000
    v = workloads.outlier_normal_f32(4, 1, 2, (n,), 0.0, 0.5, 1e-3, 50.0)
    base = workloads.normal_f32(4, 1, (n,), 0.0, 0.5)
    boosted = np.count_nonzero(v != base)
    assert 0.8e-3 * n < boosted < 1.2e-3 * n
    i = np.flatnonzero(v != base)
    assert np.allclose(v[i], base[i] * 50.0, rtol=1e-6)


def test_moe_routing_layout():
    T, ne, k = 64, 16, 4
    d = workloads.moe_inputs(5, T, 32, ne, k)
    idx, gate, ex = d["idx"].numpy(), d["gate"].numpy(), d["expert"].numpy()
    assert sorted(idx.tolist()) == list(range(T * k))          # a permutation of the rows
    assert np.allclose(gate.reshape(T, k).sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(gate.reshape(T, k), axis=1) <= 0)    # picks in descending logit order
    for t in range(T):
        assert len(set(ex[t * k:(t + 1) * k])) == k            # distinct experts per token
    # expert-major placement, (t, j) ascending inside an expert
    order = np.argsort(idx)
    keys = [(ex[i], i // k, i % k) for i in order]
    assert keys == sorted(keys)


def test_workload_shapes():
    t = workloads.tiny()
    assert t["residual"].shape == (16, 256) and len(t["partials"]) == 2
    assert t["partials"][0].dtype == torch.bfloat16 and t["weight"].dtype == torch.float32
    assert workloads.MOE_SLICE == (768, 256)
