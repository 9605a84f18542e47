"""Seeded input generators: determinism, rounding, and the workload structure."""

import numpy as np
import pytest
import torch

from rls_associative_memory_amd.inputs import (WORKLOADS, bf16_bits, get_workload, make_inputs,
                                               make_stream, round_to_bf16)


def test_round_to_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.3895314e38], dtype=np.float32),
    ])
    # exact ties: the low 16 bits are 0x8000
    ties = (rng.integers(0, 2 ** 31, 1000, dtype=np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32)])
    x = x[np.isfinite(x) | np.isinf(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    got = round_to_bf16(x)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    np.testing.assert_array_equal(bf16_bits(got), torch.from_numpy(got).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_streams_deterministic_and_independent(name):
    w = get_workload(name).resized(T=64)
    a = make_stream(w, 0)
    b = make_stream(w, 0)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
        assert x.dtype == np.float32 and x.shape == (64, w.d)
    if w.streams > 1:
        c = make_stream(w, w.streams - 1)
        assert not np.array_equal(a[0], c[0])
    if w.dtype == "bf16":
        for x in a:
            np.testing.assert_array_equal(round_to_bf16(x), x)


def test_stacked_equals_per_stream():
    w = get_workload("iid_t4096_d64").resized(B=1, H=3, T=32)
    q, k, v, u = make_inputs(w)
    assert q.shape == (3, 32, 64)
    for s in range(3):
        for full, one in zip((q, k, v, u), make_stream(w, s)):
            np.testing.assert_array_equal(full[s], one)


def test_mqar_layout():
    w = get_workload("mqar_t512_d32")
    q, k, v, u = make_stream(w, 5)
    n = w.n_pairs
    np.testing.assert_array_equal(u, k)
    np.testing.assert_allclose(np.linalg.norm(k[:n], axis=1), 1.0, rtol=1e-6)
    np.testing.assert_allclose(np.linalg.norm(v[:n], axis=1), 1.0, rtol=1e-6)
    # each key is queried exactly once, at a position after all writes
    hits = []
    for i in range(n):
        pos = np.where(np.all(q == k[i], axis=1))[0]
        assert len(pos) == 1 and pos[0] >= n
        hits.append(pos[0])
    assert len(set(hits)) == n


def test_noisy_u_layout():
    w = get_workload("crossover_t43008_d128").resized(T=128)
    q, k, v, u = make_stream(w, 1)
    diff = u.astype(np.float64) - k
    assert 0.05 < diff.std() < 0.2
